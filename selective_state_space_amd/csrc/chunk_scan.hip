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

// LDS image of one (b, h, chunk) unit, every MFMA operand stored in fragment
// order (16 bytes per lane, lane-linear), so each operand is one
// conflict-free ds_read_b128 at a constant offset.
template <int L, int N>
struct ScanSmem {
    static constexpr int NK = N / 32, NS = L / 32;
    static constexpr int NBUF = 3;          // B ring: slab js in buffer js % 3
    float G[L], V[L], DT[L];
    uint4 XF[NS][4][64];                    // x^T fragments: slab js, p = 4m + s
    union {
        uint4 HF[NK][4][64];                // h_prev fragments (inter phase only)
        uint4 BF[NBUF][2][NK][64];          // B fragments: buffer, 16-token block u, n-step kn
    };
};
static_assert(sizeof(uint4[4][4][64]) <= sizeof(uint4[3][2][4][64]), "h_prev fits the B ring");

template <int L, int N, bool RAGGED>
__device__ __forceinline__ void chunk_scan_unit(
    ScanSmem<L, N> &sm, const uint16_t *__restrict__ xb, const uint16_t *__restrict__ bb,
    const uint16_t *__restrict__ cb, const float *__restrict__ Gp, const float *__restrict__ Dp,
    const uint16_t *__restrict__ hp, float *__restrict__ yb, float Dh, int32_t nvalid,
    int32_t XR, int32_t BR) {
    constexpr int NB = L / 16;       // 16-row blocks
    constexpr int RBW = NB / 4;      // row blocks per wavefront (1 when L = 64)
    constexpr int NK = N / 32;       // K steps over n
    constexpr int NS = L / 32;       // 32-token slabs
    constexpr int BPL = (2 * NK + 3) / 4;  // B-slab pieces per thread
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;
    const int m = lane & 15, q = lane >> 4;
    auto valid = [&](int tl) { return !RAGGED || tl < nvalid; };

    // ---- staging, all global loads issued before the LDS writes ----
    // x^T fragments of slabs js = w, w+4, ...: K slot r -> token
    // 32 js + (r < 4 ? 0 : 16) + 4q + (r & 3), column m of MFMA s -> p = 4m + s
    constexpr int XSW = (NS + 3) / 4;
    uint2 xr[XSW][8];
#pragma unroll
    for (int k = 0; k < XSW; ++k) {
        const int js = w + 4 * k;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int tl = 32 * js + ((r < 4) ? 0 : 16) + 4 * q + (r & 3);
            xr[k][r] = (js < NS && valid(tl))
                           ? *reinterpret_cast<const uint2 *>(xb + tl * XR + 4 * m)
                           : make_uint2(0u, 0u);
        }
    }
    constexpr int HPL = (NK * 4 + 3) / 4;   // h_prev pieces per thread
    uint4 hv[HPL];
#pragma unroll
    for (int k = 0; k < HPL; ++k) {
        const int pc = w + 4 * k, kn = pc >> 2, s = pc & 3;
        hv[k] = (pc < NK * 4) ? *reinterpret_cast<const uint4 *>(hp + (4 * m + s) * N + 32 * kn + 8 * q)
                              : make_uint4(0u, 0u, 0u, 0u);
    }
    auto bslab_load = [&](int js, uint4 (&v)[BPL]) {
#pragma unroll
        for (int k = 0; k < BPL; ++k) {
            const int pc = w + 4 * k, u = pc / NK, kn = pc % NK;
            const int tl = 32 * js + 16 * u + m;
            v[k] = (pc < 2 * NK && valid(tl))
                       ? *reinterpret_cast<const uint4 *>(bb + tl * BR + 32 * kn + 8 * q)
                       : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto bslab_store = [&](int buf, const uint4 (&v)[BPL]) {
#pragma unroll
        for (int k = 0; k < BPL; ++k) {
            const int pc = w + 4 * k;
            if (pc < 2 * NK) sm.BF[buf][pc / NK][pc % NK][lane] = v[k];
        }
    };
    uint4 bv0[BPL];
    bslab_load(0, bv0);
    // C rows of this wavefront's row blocks I_k = w + 4k (rows 16 I_k + m,
    // n = 32 kn + 8q .. +7): A operand of the inter product and B operand of
    // the C B^T tiles, kept in registers for the whole chunk.
    uint4 cf[RBW][NK];
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
        const int tl = 16 * (w + 4 * k) + m;
#pragma unroll
        for (int kn = 0; kn < NK; ++kn)
            cf[k][kn] = valid(tl) ? *reinterpret_cast<const uint4 *>(cb + tl * BR + 32 * kn + 8 * q)
                                  : make_uint4(0u, 0u, 0u, 0u);
    }
    // G, dt and V_j = exp2(G_a - G_j) dt_j, a = the last token of j's
    // 16-block (exponent <= 0): the column factor of the decay between blocks.
    if (tid < L) {
        const float gj = Gp[tid];
        const float dj = Dp[tid];
        sm.G[tid] = gj;
        sm.DT[tid] = dj;
        sm.V[tid] = fast_exp2(Gp[tid | 15] - gj) * dj;
    }
#pragma unroll
    for (int k = 0; k < XSW; ++k) {
        const int js = w + 4 * k;
        if (js < NS) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint4 v;
                uint32_t *vw = reinterpret_cast<uint32_t *>(&v);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const uint32_t a0 = (s < 2) ? xr[k][2 * rr].x : xr[k][2 * rr].y;
                    const uint32_t a1 = (s < 2) ? xr[k][2 * rr + 1].x : xr[k][2 * rr + 1].y;
                    vw[rr] = (s & 1) ? pair_hi(a0, a1) : pair_lo(a0, a1);
                }
                sm.XF[js][s][lane] = v;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < HPL; ++k) {
        const int pc = w + 4 * k;
        if (pc < NK * 4) sm.HF[pc >> 2][pc & 3][lane] = hv[k];
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
            const bf16x8 hf = as_bf16x8(sm.HF[kn][s][lane]);
#pragma unroll
            for (int k = 0; k < RBW; ++k)
                acc[k][s] = mfma16x16x32(as_bf16x8(cf[k][kn]), hf, acc[k][s]);
        }
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
        const float4 gi = *reinterpret_cast<const float4 *>(&sm.G[16 * (w + 4 * k) + 4 * q]);
        const float sc[4] = {fast_exp2(gi.x), fast_exp2(gi.y), fast_exp2(gi.z), fast_exp2(gi.w)};
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[k][s][e] *= sc[e];
    }

    // h_prev fragments are dead: the B ring takes their place.  Slab 0 goes
    // in now, slab 1 stays in registers until the end of step 0, and each
    // step loads the slab two ahead, so a B load has two steps to land.
    __syncthreads();
    bslab_store(0, bv0);
    uint4 nb1[BPL];
    if (NS > 1) bslab_load(1, nb1);
    __syncthreads();

    // ---- intra: 32-token slabs in lockstep ----
    for (int js = 0; js < NS; ++js) {
        const int buf = js % 3;
        uint4 nb2[BPL];
        if (js + 2 < NS) bslab_load(js + 2, nb2);
        bf16x8 xf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) xf[s] = as_bf16x8(sm.XF[js][s][lane]);
        float4 vj[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
            vj[u] = *reinterpret_cast<const float4 *>(&sm.V[32 * js + 16 * u + 4 * q]);
#pragma unroll
        for (int k = 0; k < RBW; ++k) {
            const int I = w + 4 * k;
            if (I < 2 * js) continue;  // no causal tile of this row block in the slab
            const float gi = sm.G[16 * I + m];   // this lane's output row i = 16I + m
            uint32_t cw[2][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int J = 2 * js + u;
                if (J > I) {
                    cw[u][0] = 0u;
                    cw[u][1] = 0u;
                    continue;
                }
                // (C B^T)^T tile: cbt[e] = C_i . B_j, j = 16J + 4q + e
                f32x4 cbt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kn = 0; kn < NK; ++kn)
                    cbt = mfma16x16x32(as_bf16x8(sm.BF[buf][u][kn][lane]), as_bf16x8(cf[k][kn]),
                                       cbt);
                float v[4];
                if (J < I) {
                    // exp2(G_i - G_j) dt_j = exp2(G_i - G_a) * V_j, a = 16J + 15
                    const float ui = fast_exp2(gi - sm.G[16 * J + 15]);
                    v[0] = cbt[0] * (vj[u].x * ui);
                    v[1] = cbt[1] * (vj[u].y * ui);
                    v[2] = cbt[2] * (vj[u].z * ui);
                    v[3] = cbt[3] * (vj[u].w * ui);
                } else {
                    // diagonal block: exact pairwise decay, causal select (j <= i)
                    const float4 gj = *reinterpret_cast<const float4 *>(&sm.G[16 * J + 4 * q]);
                    const float4 dj = *reinterpret_cast<const float4 *>(&sm.DT[16 * J + 4 * q]);
                    const float gjv[4] = {gj.x, gj.y, gj.z, gj.w};
                    const float djv[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float val = cbt[e] * fast_exp2(fminf(gi - gjv[e], 0.f)) * djv[e];
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
        if (js + 1 < NS) bslab_store((js + 1) % 3, nb1);
#pragma unroll
        for (int k = 0; k < BPL; ++k) nb1[k] = nb2[k];
        __syncthreads();
    }

    // ---- y = acc + D x (x from this lane's own fragments), fp32 ----
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
        const int I = w + 4 * k;
        // token il = 16I + 4q + e sits in K slot e + 4 (I & 1) of this lane's
        // fragment of slab I/2: words (x, y) hold slots 0..3, (z, w) slots 4..7
        uint2 xw[4];
        const bool odd = I & 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 f = sm.XF[I >> 1][s][lane];
            xw[s] = odd ? make_uint2(f.z, f.w) : make_uint2(f.x, f.y);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int il = 16 * I + 4 * q + e;
            if (valid(il)) {
                float xv[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint32_t wd = (e < 2) ? xw[s].x : xw[s].y;
                    xv[s] = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
                }
                *reinterpret_cast<float4 *>(yb + il * XR + 4 * m) =
                    make_float4(acc[k][0][e] + Dh * xv[0], acc[k][1][e] + Dh * xv[1],
                                acc[k][2][e] + Dh * xv[2], acc[k][3][e] + Dh * xv[3]);
            }
        }
    }
}

template <int L, int N>
__global__ __launch_bounds__(256, 2) void chunk_scan_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const uint16_t *__restrict__ Cm, const float *__restrict__ D, const float *__restrict__ Gws,
    const float *__restrict__ DTws, const uint16_t *__restrict__ hprev, float *__restrict__ y,
    int64_t T, int32_t H, int32_t G, int32_t nc, uint32_t nblk) {
    constexpr int P = 64;
    __shared__ ScanSmem<L, N> sm;
    const uint32_t lid = xcd_remap(blockIdx.x, nblk);
    const int32_t h = lid % H;
    const int32_t c = (lid / H) % nc;
    const int64_t b = lid / ((uint32_t)H * nc);
    const int32_t g = h / (H / G);
    const int64_t t0 = (int64_t)c * L;
    const int64_t bhc = ((int64_t)b * H + h) * nc + c;
    const int64_t xrow0 = ((b * T + t0) * H + h) * P;      // x, y: token stride H * P
    const int64_t brow0 = ((b * T + t0) * G + g) * N;      // B, C: token stride G * N
    const int32_t XR = H * P, BR = G * N;
    const int64_t rem = T - t0;
    const int32_t nvalid = rem < L ? (int32_t)rem : L;
    if (nvalid == L)
        chunk_scan_unit<L, N, false>(sm, x + xrow0, Bm + brow0, Cm + brow0, Gws + bhc * L,
                                     DTws + bhc * L, hprev + bhc * (int64_t)(P * N), y + xrow0,
                                     D[h], nvalid, XR, BR);
    else
        chunk_scan_unit<L, N, true>(sm, x + xrow0, Bm + brow0, Cm + brow0, Gws + bhc * L,
                                    DTws + bhc * L, hprev + bhc * (int64_t)(P * N), y + xrow0,
                                    D[h], nvalid, XR, BR);
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
