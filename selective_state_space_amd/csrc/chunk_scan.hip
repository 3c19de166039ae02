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
// per (b, h, chunk), heads fastest and kept on one XCD so the group's B and C
// come from L2.  Wavefront w owns the 16-row blocks I = w, w+4, ... of the
// chunk and keeps their C rows in registers (A operand of the inter product,
// B operand of the C B^T tiles).  h_prev, G, dt and the column factors V are
// staged in LDS once; B and x go through LDS in 32-token slabs, the next slab
// loaded while the current one is used (all wavefronts in lockstep).
//   1. inter: acc = C h_prev^T (K = N); output column m of MFMA s is p = 4m+s.
//      Rows are then scaled by exp2(G_i).
//   2. intra, per slab: two 16x16 tiles of (C B^T)^T = B C^T per row block
//      (A = B rows from LDS).  The accumulator layout of a transposed tile
//      (lane m: column i, rows j = 4q..4q+3) is a 4-element K slice of the A
//      operand for row i, so the drain -- times exp2(G_i - G_j) dt_j, select
//      j <= i, round to bf16 -- leaves the A operand of the second product in
//      place, with no LDS round trip.  The matching B operand (x rows of the
//      same tokens, 4 p per lane) is transposed in registers.  Tiles above the
//      diagonal are skipped.  Below the diagonal the decay factors through
//      the last token a of the column block: exp2(G_i - G_j) = exp2(G_i - G_a)
//      * exp2(G_a - G_j), both exponents <= 0, so a tile needs one exp2 per
//      lane (V_j = exp2(G_a - G_j) dt_j is staged per token).  Diagonal tiles
//      use the exact pairwise exponent with a causal select.
//   3. y = acc + D x, written fp32 (16 bytes a lane and row).
//
// fp32 path (VALU): one workgroup per (b, h, chunk), 16-row tiles: the
// decayed, masked C B^T rows are built in LDS, then each thread forms y for
// one p and four rows.

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

template <int L, int N>
__global__ __launch_bounds__(256, 2) void chunk_scan_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const uint16_t *__restrict__ Cm, const float *__restrict__ D, const float *__restrict__ Gws,
    const float *__restrict__ DTws, const uint16_t *__restrict__ hprev, float *__restrict__ y,
    int64_t T, int32_t H, int32_t G, int32_t nc, uint32_t nblk) {
    constexpr int P = 64;
    constexpr int NB = L / 16;       // 16-row blocks
    constexpr int RBW = NB / 4;      // row blocks per wavefront
    constexpr int NK = N / 32;       // K steps over n
    constexpr int NS = L / 32;       // 32-token slabs
    constexpr int HS = N + 8;        // padded LDS row strides (bf16 elements)
    constexpr int XS = P + 8;
    __shared__ float Gs[L], Vs[L], DTs[L];
    __shared__ __attribute__((aligned(16))) uint16_t Hs[P * HS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][32 * HS];
    __shared__ __attribute__((aligned(16))) uint16_t Xs[2][32 * XS];

    const uint32_t lid = xcd_remap(blockIdx.x, nblk);
    const int32_t h = lid % H;
    const int32_t c = (lid / H) % nc;
    const int64_t b = lid / ((uint32_t)H * nc);
    const int32_t g = h / (H / G);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m = lane & 15, q = lane >> 4;

    const int64_t bhc = ((int64_t)b * H + h) * nc + c;
    const float *Gp = Gws + bhc * L;
    const float *Dp = DTws + bhc * L;
    const uint16_t *Hp = hprev + bhc * (int64_t)(P * N);
    const float Dh = D[h];
    const int64_t t0 = (int64_t)c * L;

    // ---- staging: G, dt, the column weights V, h_prev, slab 0 of B and x ----
    // V_j = exp2(G_a - G_j) dt_j with a = the last token of j's 16-block
    // (exponent <= 0): the column factor of the decay between blocks.
    if (tid < L) {
        const float gj = Gp[tid];
        const float dj = Dp[tid];
        Gs[tid] = gj;
        DTs[tid] = dj;
        Vs[tid] = fast_exp2(Gp[(tid | 15)] - gj) * dj;
    }
    for (int e = tid; e < P * (N / 8); e += 256) {
        const int r = e / (N / 8), cc = (e % (N / 8)) * 8;
        *reinterpret_cast<uint4 *>(&Hs[r * HS + cc]) =
            *reinterpret_cast<const uint4 *>(Hp + r * N + cc);
    }
    // slab staging: B rows (N/8 16-byte pieces each) then x rows (8 pieces each)
    constexpr int BPC = 32 * (N / 8);         // B pieces per slab
    constexpr int XPC = 32 * 8;               // x pieces per slab
    constexpr int PPT = (BPC + XPC) / 256;    // pieces per thread
    static_assert((BPC + XPC) % 256 == 0, "slab pieces must spread evenly");
    auto slab_load = [&](int js, uint4 (&v)[PPT]) {
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int e = tid + 256 * k;
            const bool isb = e < BPC;
            const int ee = isb ? e : e - BPC;
            const int r = isb ? ee / (N / 8) : ee / 8;
            const int cc = isb ? (ee % (N / 8)) * 8 : (ee % 8) * 8;
            const int64_t tok = t0 + 32 * js + r;
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (tok < T)
                val = isb ? *reinterpret_cast<const uint4 *>(Bm + ((b * T + tok) * G + g) * N + cc)
                          : *reinterpret_cast<const uint4 *>(x + ((b * T + tok) * H + h) * P + cc);
            v[k] = val;
        }
    };
    auto slab_store = [&](int buf, const uint4 (&v)[PPT]) {
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int e = tid + 256 * k;
            const bool isb = e < BPC;
            const int ee = isb ? e : e - BPC;
            if (isb)
                *reinterpret_cast<uint4 *>(&Bs[buf][(ee / (N / 8)) * HS + (ee % (N / 8)) * 8]) = v[k];
            else
                *reinterpret_cast<uint4 *>(&Xs[buf][(ee / 8) * XS + (ee % 8) * 8]) = v[k];
        }
    };
    {
        uint4 v[PPT];
        slab_load(0, v);
        slab_store(0, v);
    }

    // C rows of this wavefront's row blocks I_k = wave + 4k (rows 16 I_k + m,
    // n = 32 kn + 8q .. +7): A operand of the inter product and B operand of
    // the C B^T tiles, kept in registers for the whole chunk.
    uint4 cf[RBW][NK];
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
        const int64_t tok = t0 + 16 * (wave + 4 * k) + m;
        const uint16_t *cp = Cm + ((b * T + tok) * G + g) * N + 8 * q;
#pragma unroll
        for (int kn = 0; kn < NK; ++kn)
            cf[k][kn] = tok < T ? *reinterpret_cast<const uint4 *>(cp + 32 * kn)
                                : make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();

    // ---- inter: acc = C h_prev^T, then rows scaled by exp2(G_i) ----
    // acc[k][s][e] = y[i = 16 I_k + 4q + e][p = 4m + s]
    f32x4 acc[RBW][4];
#pragma unroll
    for (int k = 0; k < RBW; ++k)
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[k][s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kn = 0; kn < NK; ++kn)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 hv = *reinterpret_cast<const uint4 *>(&Hs[(4 * m + s) * HS + 32 * kn + 8 * q]);
#pragma unroll
            for (int k = 0; k < RBW; ++k)
                acc[k][s] = mfma16x16x32(as_bf16x8(cf[k][kn]), as_bf16x8(hv), acc[k][s]);
        }
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
        const int i0 = 16 * (wave + 4 * k) + 4 * q;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float sc = fast_exp2(Gs[i0 + e]);
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[k][s][e] *= sc;
        }
    }

    // ---- intra: 32-token slabs in lockstep, next slab loaded during this one ----
    for (int js = 0; js < NS; ++js) {
        const int buf = js & 1;
        uint4 nxt[PPT];
        if (js + 1 < NS) slab_load(js + 1, nxt);

        // x rows of the slab as B operands: K slot r -> token (r < 4 ? 0 : 16) + 4q + (r & 3),
        // column m of MFMA s -> p = 4m + s (transposed in registers)
        bf16x8 xf[4];
        {
            uint2 xr[8];
#pragma unroll
            for (int r = 0; r < 8; ++r)
                xr[r] = *reinterpret_cast<const uint2 *>(
                    &Xs[buf][((r < 4 ? 0 : 16) + 4 * q + (r & 3)) * XS + 4 * m]);
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
                xf[s] = as_bf16x8(v);
            }
        }
#pragma unroll
        for (int k = 0; k < RBW; ++k) {
            const int I = wave + 4 * k;
            if (I < 2 * js) continue;  // wave-uniform: no causal tile in this slab
            const int icol = 16 * I + m;             // this lane's output row i
            const float gi = Gs[icol];
            uint32_t cw[2][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int J = 2 * js + u;
                if (J > I) {
                    cw[u][0] = 0u;
                    cw[u][1] = 0u;
                    continue;
                }
                // (C B^T)^T tile: cbt[e] = C_i . B_j, i = 16I + m, j = 16J + 4q + e
                f32x4 cbt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kn = 0; kn < NK; ++kn) {
                    const uint4 bv = *reinterpret_cast<const uint4 *>(
                        &Bs[buf][(16 * u + m) * HS + 32 * kn + 8 * q]);
                    cbt = mfma16x16x32(as_bf16x8(bv), as_bf16x8(cf[k][kn]), cbt);
                }
                const int j0 = 16 * J + 4 * q;
                float v[4];
                if (J < I) {
                    // exp2(G_i - G_j) dt_j = exp2(G_i - G_a) * V_j, a = 16J + 15
                    const float ui = fast_exp2(gi - Gs[16 * J + 15]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = cbt[e] * (Vs[j0 + e] * ui);
                } else {
                    // diagonal block: exact pairwise decay, causal select (j <= i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float d = fminf(gi - Gs[j0 + e], 0.f);
                        const float val = cbt[e] * fast_exp2(d) * DTs[j0 + e];
                        v[e] = (4 * q + e <= m) ? val : 0.f;
                    }
                }
                cw[u][0] = pack_bf16x2(v[0], v[1]);
                cw[u][1] = pack_bf16x2(v[2], v[3]);
            }
            const bf16x8 af = as_bf16x8(make_uint4(cw[0][0], cw[0][1], cw[1][0], cw[1][1]));
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[k][s] = mfma16x16x32(af, xf[s], acc[k][s]);
        }
        if (js + 1 < NS) slab_store(buf ^ 1, nxt);
        __syncthreads();
    }

    // ---- y = acc + D x, fp32, 16 bytes per lane and row ----
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t tok = t0 + 16 * (wave + 4 * k) + 4 * q + e;
            if (tok < T) {
                const int64_t off = ((b * T + tok) * H + h) * P + 4 * m;
                const uint2 xv = *reinterpret_cast<const uint2 *>(x + off);
                const float4 o = make_float4(acc[k][0][e] + Dh * bf16_lo(xv.x),
                                             acc[k][1][e] + Dh * bf16_hi(xv.x),
                                             acc[k][2][e] + Dh * bf16_lo(xv.y),
                                             acc[k][3][e] + Dh * bf16_hi(xv.y));
                *reinterpret_cast<float4 *>(y + off) = o;
            }
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
                           DTws, (const uint16_t *)hprev, (float *)y, s.T, (int32_t)s.H,
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
