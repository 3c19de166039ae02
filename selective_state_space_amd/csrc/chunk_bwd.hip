// The backward of the chunked forward: gradients of L = sum(dy . y) +
// sum(dfinal . final) with respect to x, dt, A, B, C, D and the initial state.
//
// the "mamba3" kernel card, section "Backward": two chunk-parallel passes around a
// reverse scan of the state adjoint, with the chunk intermediates recomputed
// rather than stored, and no floating-point atomics (every output element has
// one owner; sums over heads and batch rows are taken in a fixed order).
// The arithmetic is the chain rule of the recurrence of "Accelerating Mamba-2
// with High-Performance Forward Pass Kernels in NVIDIA CUDA Tile", section
// "Mamba-2 architecture", in the chunked form of the same section.  Per
// (b, h), chunk c, chunk-local log-decay G (log2 units here) and the adjoint
// ghat_c of the state leaving chunk c (ghat of the last chunk = dfinal):
//
//   dSp_c   = sum_k exp(G_k) dy_k (outer) C_k                    (bwd_dstate)
//   ghat_{c-1} = dSp_c + exp(G_last) ghat_c; dinit = ghat_{-1}    (bwd_passing)
//   CB(k,j) = C_k . B_j                                           (bwd_cb)
//   U_i = sum_{k>=i} exp(G_k-G_i) CB(k,i) dy_k + exp(G_last-G_i) ghat_c B_i
//        (the state adjoint g_i times B_i);  dx_i = D dy_i + dt_i U_i
//   Y_i = exp(G_i) h_prev C_i + sum_{j<=i} exp(G_i-G_j) CB(i,j) dt_j x_j
//   r_i = dy_i . Y_i - dt_i x_i . U_i                              (bwd_dx)
//   M(k,j) = sum_h [k>=j] exp(G_k-G_j) dt_j (dy_k . x_j)
//   dC_k = sum_j M(k,j) B_j + sum_h exp(G_k) h_prev^T dy_k
//   dB_j = sum_k M(k,j) C_k + sum_h dt_j exp(G_last-G_j) ghat_c^T x_j
//                                     (bwd_dbdc; bwd_dc_mfma and bwd_db_mfma)
//   s_t  = <dfinal, final> + sum_{t'>=t} r_t'  (over the whole sequence)
//   ddt_t = x_t . U_t + A s_t;  dA = sum dt_t s_t;  dD = sum dy_t . x_t
//                                                   (bwd_scalars, bwd_heads)
// The identity behind s_t: with g_t the state adjoint, <g_t, exp(A dt_t)
// h_{t-1}> = dy_t . (h_t C_t) - dt_t x_t . (g_t B_t) + <g_{t+1}, exp(A dt_{t+1}) h_t>,
// so the decay part of the step gradient is a reverse running sum of per-token
// scalars and never needs a per-token state.
//
// bf16 io runs bwd_dx, dC and dB on bf16 MFMA with fp32 operands split into
// two or three bf16 terms; fp32 io runs fp32 SIMT versions that stage operand
// tiles into LDS and accumulate small register tiles per thread.  h_prev is
// read in fp32 (recomputed with fp32 stores, by the one-pass state kernel or
// by chunk_state + state_passing): the decay gradients sum per-token products
// with it over the whole sequence, and bf16's rounding of it would not average
// out there.  Where the forward takes the one-pass form, the same kernel also
// runs the state adjoint scan (dSp and the reverse scan in one pass, chunks
// last to first); bwd_dstate and bwd_passing serve the other shapes.

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int P = 64;
constexpr int KT = 32;        // K-tile of the staged products
constexpr int LD = 68;        // LDS row pitch in floats (16-byte aligned, 2-way at worst)

template <typename T>
__device__ __forceinline__ float ld1(const T *p);
template <>
__device__ __forceinline__ float ld1<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float ld1<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

// acc[TM][TN] += sum_{k < KT} As[k][m0 + i] * Bs[k][n0 + j]
template <int TM, int TN>
__device__ __forceinline__ void mm_acc(float (&acc)[TM][TN], const float *As, int lda,
                                       const float *Bs, int ldb, int m0, int n0) {
#pragma unroll 4
    for (int k = 0; k < KT; ++k) {
        float a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; i += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(As + k * lda + m0 + i);
            a[i] = v.x; a[i + 1] = v.y; a[i + 2] = v.z; a[i + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < TN; j += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(Bs + k * ldb + n0 + j);
            b[j] = v.x; b[j + 1] = v.y; b[j + 2] = v.z; b[j + 3] = v.w;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
}

// ---- bf16 operand helpers shared by the MFMA kernels below -----------------
constexpr int SP = P + 16;    // LDS row pitch (bf16) of the staged [row][p] tiles: 40
                              // words (a 36-word pitch left the 16-byte MFMA operand
                              // reads with bank conflicts, measured)

__device__ __forceinline__ uint4 pack8(const float (&v)[8]) {
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
}
// v = hi + lo with hi = bf16(v), lo = bf16(v - hi)
__device__ __forceinline__ void split8(const float (&v)[8], uint4 &hi, uint4 &lo) {
    hi = pack8(v);
    const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
    float r[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = v[2 * i] - bf16_lo(hw[i]);
        r[2 * i + 1] = v[2 * i + 1] - bf16_hi(hw[i]);
    }
    lo = pack8(r);
}
__device__ __forceinline__ void split1(float v, uint16_t &hi, uint16_t &lo) {
    const uint32_t h = pack_bf16x2(v, 0.f) & 0xffffu;
    hi = (uint16_t)h;
    lo = (uint16_t)(pack_bf16x2(v - __uint_as_float(h << 16), 0.f) & 0xffffu);
}
// three bf16 terms: v = s0 + s1 + s2 up to about 2^-27 of v
__device__ __forceinline__ void split8x3(const float (&v)[8], uint4 &s0, uint4 &s1, uint4 &s2) {
    float r[8];
    s0 = pack8(v);
    const uint32_t a[4] = {s0.x, s0.y, s0.z, s0.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = v[2 * i] - bf16_lo(a[i]);
        r[2 * i + 1] = v[2 * i + 1] - bf16_hi(a[i]);
    }
    s1 = pack8(r);
    const uint32_t bq[4] = {s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] -= bf16_lo(bq[i]);
        r[2 * i + 1] -= bf16_hi(bq[i]);
    }
    s2 = pack8(r);
}
__device__ __forceinline__ void split1x3(float v, uint16_t &s0, uint16_t &s1, uint16_t &s2) {
    const uint32_t a = pack_bf16x2(v, 0.f) & 0xffffu;
    const float r1 = v - __uint_as_float(a << 16);
    const uint32_t bq = pack_bf16x2(r1, 0.f) & 0xffffu;
    const float r2 = r1 - __uint_as_float(bq << 16);
    s0 = (uint16_t)a;
    s1 = (uint16_t)bq;
    s2 = (uint16_t)(pack_bf16x2(r2, 0.f) & 0xffffu);
}
// the two 16-bit halves of a word: lo = the element of the even index
__device__ __forceinline__ uint32_t pair16(uint32_t lo, uint32_t hi) { return (lo & 0xffffu) | (hi << 16); }
// split1x3 / split1 of two values at once, one paired conversion per term
__device__ __forceinline__ void split2x3(float a, float b, uint32_t &s0, uint32_t &s1, uint32_t &s2) {
    s0 = pack_bf16x2(a, b);
    const float ra = a - bf16_lo(s0), rb = b - bf16_hi(s0);
    s1 = pack_bf16x2(ra, rb);
    s2 = pack_bf16x2(ra - bf16_lo(s1), rb - bf16_hi(s1));
}
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pack_bf16x2(a, b);
    lo = pack_bf16x2(a - bf16_lo(hi), b - bf16_hi(hi));
}

// ---- bwd_dstate: dSp[b,h,c] = sum_k exp2(G_k) dy_k (outer) C_k, [P][N] ------
template <int L, int N, typename Tio>
__global__ __launch_bounds__(256) void bwd_dstate_kernel(const float *__restrict__ dy,
                                                         const Tio *__restrict__ C,
                                                         const float *__restrict__ Gws,
                                                         float *__restrict__ dS, int64_t T,
                                                         int32_t H, int32_t G, int32_t nc) {
    constexpr int TN = N / 16;
    __shared__ __align__(16) float As[KT * LD];
    __shared__ __align__(16) float Bs[KT * (N + 4)];
    // logical order (b, c, g, head) with the head fastest, consecutive ids on
    // one XCD: the heads of a group share the chunk's C rows in that L2
    const int64_t blk = xcd_remap(blockIdx.x, gridDim.x);
    const int hpg = H / G;
    const int32_t h = (int32_t)((blk / hpg) % G) * hpg + (int32_t)(blk % hpg);
    const int32_t g = h / hpg;
    const int32_t c = (int32_t)((blk / H) % nc);
    const int64_t b = blk / H / nc;
    const int64_t unit = (b * H + h) * nc + c;
    const int tid = threadIdx.x;
    const int p0 = 4 * (tid >> 4), n0 = TN * (tid & 15);
    const float *Gc = Gws + unit * L;
    float acc[4][TN] = {};
    for (int k0 = 0; k0 < L; k0 += KT) {
        __syncthreads();
        for (int e = tid; e < KT * P; e += 256) {          // dy rows, scaled
            const int kk = e / P, p = e % P;
            const int64_t t = (int64_t)c * L + k0 + kk;
            As[kk * LD + p] = t < T ? dy[((b * T + t) * H + h) * P + p] * fast_exp2(Gc[k0 + kk]) : 0.f;
        }
        for (int e = tid; e < KT * N; e += 256) {
            const int kk = e / N, n = e % N;
            const int64_t t = (int64_t)c * L + k0 + kk;
            Bs[kk * (N + 4) + n] = t < T ? ld1(C + ((b * T + t) * G + g) * N + n) : 0.f;
        }
        __syncthreads();
        mm_acc<4, TN>(acc, As, LD, Bs, N + 4, p0, n0);
    }
    float *o = dS + unit * (int64_t)(P * N);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; j += 4)
            *reinterpret_cast<float4 *>(o + (p0 + i) * N + n0 + j) =
                make_float4(acc[i][j], acc[i][j + 1], acc[i][j + 2], acc[i][j + 3]);
}

// ---- bwd_passing: reverse scan of the state adjoint, in place over dSp ------
// The slot of chunk c ends holding ghat_c (the adjoint of the state leaving c).
template <int L, int N>
__global__ __launch_bounds__(256) void bwd_passing_kernel(float *__restrict__ dS,
                                                          const float *__restrict__ Gws,
                                                          const float *__restrict__ dfin,
                                                          const float *__restrict__ fin,
                                                          float *__restrict__ dinit,
                                                          double *__restrict__ bnd, int32_t nc) {
    constexpr int E = P * N / 256;                 // elements per thread
    __shared__ double red[256];
    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t off = bh * (int64_t)(P * N) + (int64_t)tid * E;
    float gh[E];
    double dot = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        gh[e] = dfin ? dfin[off + e] : 0.f;
        if (dfin) dot += (double)gh[e] * (double)fin[off + e];
    }
    for (int c = nc - 1; c >= 0; --c) {
        float *slot = dS + (bh * nc + c) * (int64_t)(P * N) + (int64_t)tid * E;
        const float a = fast_exp2(Gws[(bh * nc + c) * L + (L - 1)]);
#pragma unroll
        for (int e = 0; e < E; e += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(slot + e);
            *reinterpret_cast<float4 *>(slot + e) =
                make_float4(gh[e], gh[e + 1], gh[e + 2], gh[e + 3]);
            gh[e] = fmaf(a, gh[e], v.x);
            gh[e + 1] = fmaf(a, gh[e + 1], v.y);
            gh[e + 2] = fmaf(a, gh[e + 2], v.z);
            gh[e + 3] = fmaf(a, gh[e + 3], v.w);
        }
    }
    if (dinit)
#pragma unroll
        for (int e = 0; e < E; ++e) dinit[off + e] = gh[e];
    red[tid] = dot;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    if (tid == 0) bnd[bh] = red[0];
}

// ---- bwd_bnd: bnd[bh] = <dfinal, final> of one (b, h) in fp64, coalesced
// 16-byte loads (the one-pass adjoint scan leaves only this of bwd_passing)
template <int N>
__global__ __launch_bounds__(256) void bwd_bnd_kernel(const float *__restrict__ dfin,
                                                      const float *__restrict__ fin,
                                                      double *__restrict__ bnd) {
    constexpr int E4 = P * N / 4 / 256;            // float4 per thread
    __shared__ double red[256];
    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const float4 *d4 = reinterpret_cast<const float4 *>(dfin + bh * (int64_t)(P * N));
    const float4 *f4 = reinterpret_cast<const float4 *>(fin + bh * (int64_t)(P * N));
    float4 dv[E4], fv[E4];
#pragma unroll
    for (int e = 0; e < E4; ++e) {
        dv[e] = d4[e * 256 + tid];
        fv[e] = f4[e * 256 + tid];
    }
    double dot = 0.0;
#pragma unroll
    for (int e = 0; e < E4; ++e)
        dot += (double)dv[e].x * fv[e].x + (double)dv[e].y * fv[e].y + (double)dv[e].z * fv[e].z +
               (double)dv[e].w * fv[e].w;
    red[tid] = dot;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    if (tid == 0) bnd[bh] = red[0];
}

__global__ __launch_bounds__(256) void fill_f64_kernel(double *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0;
}

// ---- bwd_cb: CB(k, j) = C_k . B_j for the 64x64 blocks on or below the diagonal
template <int L, int N, typename Tio>
__global__ __launch_bounds__(256) void bwd_cb_kernel(const Tio *__restrict__ B,
                                                     const Tio *__restrict__ C,
                                                     float *__restrict__ CB, int64_t T,
                                                     int32_t G, int32_t nc) {
    constexpr int NB = L / 64, NTRI = NB * (NB + 1) / 2;
    __shared__ __align__(16) float As[KT * LD];
    __shared__ __align__(16) float Bs[KT * LD];
    const int64_t blk = blockIdx.x;
    int tri = (int)(blk % NTRI);
    const int64_t bcg = blk / NTRI;                // (b*nc + c)*G + g
    const int32_t g = (int32_t)(bcg % G);
    const int64_t bc = bcg / G;
    const int32_t c = (int32_t)(bc % nc);
    const int64_t b = bc / nc;
    int kb = 0;
    while (tri > kb) { tri -= kb + 1; ++kb; }
    const int jb = tri;                             // jb <= kb
    const int tid = threadIdx.x;
    const int m0 = 4 * (tid >> 4), n0 = 4 * (tid & 15);
    float acc[4][4] = {};
    for (int q0 = 0; q0 < N; q0 += KT) {
        __syncthreads();
        for (int e = tid; e < KT * 64; e += 256) {
            const int r = e / KT, q = e % KT;       // token row r, state index q
            const int64_t tk = (int64_t)c * L + 64 * kb + r, tj = (int64_t)c * L + 64 * jb + r;
            As[q * LD + r] = tk < T ? ld1(C + ((b * T + tk) * G + g) * N + q0 + q) : 0.f;
            Bs[q * LD + r] = tj < T ? ld1(B + ((b * T + tj) * G + g) * N + q0 + q) : 0.f;
        }
        __syncthreads();
        mm_acc<4, 4>(acc, As, LD, Bs, LD, m0, n0);
    }
    float *o = CB + bcg * (int64_t)(L * L) + (int64_t)(64 * kb + m0) * L + 64 * jb + n0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4 *>(o + i * L) =
            make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
}

// ---- bwd_cb_mfma (bf16 io): C B^T and its transpose as three bf16 terms each,
// [term][bcg][row][col], for the 64x64 blocks on or below the diagonal (the
// diagonal blocks whole).  B and C are exact bf16, so the MFMA's fp32 sums are
// the fp32 products' sums.  Wavefront w takes rows k = 64 kb + 16 w .. +15
// against the four 16-column tiles of block jb; each tile is formed both ways
// (C B^T and B C^T), so that each layout leaves the D registers as 4
// consecutive elements of one row per lane (8-byte stores per term).
template <int L, int N>
__global__ __launch_bounds__(256) void bwd_cb_mfma_kernel(const uint16_t *__restrict__ B,
                                                          const uint16_t *__restrict__ C,
                                                          uint16_t *__restrict__ CB3,
                                                          uint16_t *__restrict__ CBT3, int64_t T,
                                                          int32_t G, int32_t nc) {
    constexpr int NB = L / 64, NTRI = NB * (NB + 1) / 2, NK = N / 32;
    const int64_t blk = blockIdx.x;
    int tri = (int)(blk % NTRI);
    const int64_t bcg = blk / NTRI;                // (b*nc + c)*G + g
    const int32_t g = (int32_t)(bcg % G);
    const int64_t bc = bcg / G;
    const int32_t c = (int32_t)(bc % nc);
    const int64_t b = bc / nc;
    int kb = 0;
    while (tri > kb) { tri -= kb + 1; ++kb; }
    const int jb = tri;                             // jb <= kb
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, q = lane >> 4;
    const int64_t tc = (int64_t)c * L;
    const int k0 = 64 * kb + 16 * w;
    // B and C rows of the chunk through buffers whose range ends at the
    // sequence end (rows past it read 0), so that every load of the block
    // goes out before any is used
    const uint32_t nvt = (uint32_t)(T - tc < L ? T - tc : L), rowb = (uint32_t)(G * N * 2);
    const int64_t row0 = ((b * T + tc) * G + g) * N;
    const auto rc = make_rsrc(C + row0, nvt * rowb), rbb = make_rsrc(B + row0, nvt * rowb);
    auto ld = [&](__amdgpu_buffer_rsrc_t r, int row, int ks) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)row * rowb + 2u * (32 * ks + 8 * q), 0, 0);
        return __builtin_bit_cast(bf16x8, v);
    };
    bf16x8 ca[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) ca[ks] = ld(rc, k0 + m, ks);
    const int64_t plane = (int64_t)gridDim.x / NTRI * L * L;   // Bt*nc*G*L*L
    const int64_t base = bcg * (int64_t)(L * L);
    bf16x8 bb[4][NK];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) bb[jt][ks] = ld(rbb, 64 * jb + 16 * jt + m, ks);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const int j0 = 64 * jb + 16 * jt;
        f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f}, dtr = d;
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
            const bf16x8 bv = bb[jt][ks];
            d = mfma16x16x32(ca[ks], bv, d);       // rows k, column j
            dtr = mfma16x16x32(bv, ca[ks], dtr);   // rows j, column k
        }
        uint32_t s0a, s1a, s2a, s0b, s1b, s2b;
        // CBT3[j = j0 + m][k = k0 + 4q .. +3]
        split2x3(d[0], d[1], s0a, s1a, s2a);
        split2x3(d[2], d[3], s0b, s1b, s2b);
        int64_t o = base + (int64_t)(j0 + m) * L + k0 + 4 * q;
        *reinterpret_cast<uint2 *>(CBT3 + o) = make_uint2(s0a, s0b);
        *reinterpret_cast<uint2 *>(CBT3 + plane + o) = make_uint2(s1a, s1b);
        *reinterpret_cast<uint2 *>(CBT3 + 2 * plane + o) = make_uint2(s2a, s2b);
        // CB3[k = k0 + m][j = j0 + 4q .. +3]
        split2x3(dtr[0], dtr[1], s0a, s1a, s2a);
        split2x3(dtr[2], dtr[3], s0b, s1b, s2b);
        o = base + (int64_t)(k0 + m) * L + j0 + 4 * q;
        *reinterpret_cast<uint2 *>(CB3 + o) = make_uint2(s0a, s0b);
        *reinterpret_cast<uint2 *>(CB3 + plane + o) = make_uint2(s1a, s1b);
        *reinterpret_cast<uint2 *>(CB3 + 2 * plane + o) = make_uint2(s2a, s2b);
    }
}

// ---- bwd_dx: dx and the per-token scalars of one (b, c, h, 64-row block) ----
template <int L, int N, typename Tio, typename Thp>
__global__ __launch_bounds__(256) void bwd_dx_kernel(
    const Tio *__restrict__ x, const Tio *__restrict__ B, const Tio *__restrict__ C,
    const float *__restrict__ D, const float *__restrict__ dy, const float *__restrict__ Gws,
    const float *__restrict__ DTws, const float *__restrict__ CB, const float *__restrict__ gh,
    const Thp *__restrict__ hprev, float *__restrict__ dx, float *__restrict__ tok, int64_t T,
    int32_t H, int32_t G, int32_t nc) {
    __shared__ __align__(16) float As[KT * LD];
    __shared__ __align__(16) float Bs[KT * LD];
    const int64_t blk = blockIdx.x;
    const int ib = (int)(blk % (L / 64));
    const int64_t unit = blk / (L / 64);            // (b*H + h)*nc + c
    const int32_t c = (int32_t)(unit % nc);
    const int64_t bh = unit / nc;
    const int64_t b = bh / H;
    const int32_t h = (int32_t)(bh % H), g = h / (H / G);
    const int64_t bcg = ((b * nc) + c) * G + g;
    const int i0 = 64 * ib;
    const int tid = threadIdx.x;
    const int m0 = 4 * (tid >> 4), n0 = 4 * (tid & 15);
    const float *Gc = Gws + unit * L, *DTc = DTws + unit * L;
    const float *CBc = CB + bcg * (int64_t)(L * L);
    const int64_t tc = (int64_t)c * L;
    const float glast = Gc[L - 1];
    float U[4][4] = {}, Y[4][4] = {};

    // U intra: sum_{k >= i} exp2(G_k - G_i) CB(k, i) dy_k
    for (int k0 = i0; k0 < L; k0 += KT) {
        __syncthreads();
        for (int e = tid; e < KT * 64; e += 256) {
            const int kk = e / 64, ii = e % 64;
            const int k = k0 + kk, i = i0 + ii;
            As[kk * LD + ii] = k >= i ? fast_exp2(Gc[k] - Gc[i]) * CBc[(int64_t)k * L + i] : 0.f;
            const int64_t t = tc + k;
            Bs[kk * LD + ii] = t < T ? dy[((b * T + t) * H + h) * P + ii] : 0.f;
        }
        __syncthreads();
        mm_acc<4, 4>(U, As, LD, Bs, LD, m0, n0);
    }
    // U inter: exp2(G_last - G_i) ghat_c B_i;  Y inter: exp2(G_i) h_prev C_i
    const float *ghc = gh + unit * (int64_t)(P * N);
    const Thp *hpc = hprev + unit * (int64_t)(P * N);
    for (int q0 = 0; q0 < N; q0 += KT) {
        __syncthreads();
        for (int e = tid; e < KT * 64; e += 256) {
            const int ii = e / KT, q = e % KT;
            const int64_t t = tc + i0 + ii;
            const float f = fast_exp2(glast - Gc[i0 + ii]);
            As[q * LD + ii] = t < T ? f * ld1(B + ((b * T + t) * G + g) * N + q0 + q) : 0.f;
            Bs[q * LD + ii] = ghc[ii * N + q0 + q];    // ii plays p here
        }
        __syncthreads();
        mm_acc<4, 4>(U, As, LD, Bs, LD, m0, n0);
        __syncthreads();
        for (int e = tid; e < KT * 64; e += 256) {
            const int ii = e / KT, q = e % KT;
            const int64_t t = tc + i0 + ii;
            const float f = fast_exp2(Gc[i0 + ii]);
            As[q * LD + ii] = t < T ? f * ld1(C + ((b * T + t) * G + g) * N + q0 + q) : 0.f;
            Bs[q * LD + ii] = ld1(hpc + ii * N + q0 + q);
        }
        __syncthreads();
        mm_acc<4, 4>(Y, As, LD, Bs, LD, m0, n0);
    }
    // Y intra: sum_{j <= i} exp2(G_i - G_j) CB(i, j) dt_j x_j
    for (int j0 = 0; j0 < i0 + 64; j0 += KT) {
        __syncthreads();
        for (int e = tid; e < KT * 64; e += 256) {
            const int ii = e / KT, jj = e % KT;
            const int i = i0 + ii, j = j0 + jj;
            As[jj * LD + ii] =
                j <= i ? fast_exp2(Gc[i] - Gc[j]) * CBc[(int64_t)i * L + j] * DTc[j] : 0.f;
        }
        for (int e = tid; e < KT * 64; e += 256) {
            const int jj = e / 64, p = e % 64;
            const int64_t t = tc + j0 + jj;
            Bs[jj * LD + p] = t < T ? ld1(x + ((b * T + t) * H + h) * P + p) : 0.f;
        }
        __syncthreads();
        mm_acc<4, 4>(Y, As, LD, Bs, LD, m0, n0);
    }
    // epilogue: dx, and x.U, dy.Y, dy.x summed over p (16 lanes share a row)
    const float Dh = D[h];
    float *tokc = tok + unit * (int64_t)L;
    const int64_t ntok = (int64_t)gridDim.x / (L / 64) * L;   // one plane of token scalars
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = i0 + m0 + e;
        const int64_t t = tc + i;
        const bool real = t < T;
        const int64_t tt = real ? t : 0;
        const float dti = DTc[i];
        float xu = 0.f, dyy = 0.f, dyx = 0.f;
        float dv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int p = n0 + s;
            const float dyv = real ? dy[((b * T + tt) * H + h) * P + p] : 0.f;
            const float xv = real ? ld1(x + ((b * T + tt) * H + h) * P + p) : 0.f;
            dv[s] = Dh * dyv + dti * U[e][s];
            xu = fmaf(xv, U[e][s], xu);
            dyy = fmaf(dyv, Y[e][s], dyy);
            dyx = fmaf(dyv, xv, dyx);
        }
        if (real)
            *reinterpret_cast<float4 *>(dx + ((b * T + t) * H + h) * P + n0) =
                make_float4(dv[0], dv[1], dv[2], dv[3]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            xu += __shfl_xor(xu, o, 64);
            dyy += __shfl_xor(dyy, o, 64);
            dyx += __shfl_xor(dyx, o, 64);
        }
        if ((tid & 15) == 0) {
            tokc[i] = xu;                            // x . U  (plane 0)
            tokc[ntok + i] = dyy - dti * xu;         // r      (plane 1)
            tokc[2 * ntok + i] = dyx;                // dy . x (plane 2)
        }
    }
}

// ---- bwd_dbdc: dC (orientation 0) or dB (orientation 1) for one 64-row block
template <int L, int N, typename Tio, typename Thp>
__global__ __launch_bounds__(256) void bwd_dbdc_kernel(
    const Tio *__restrict__ x, const Tio *__restrict__ B, const Tio *__restrict__ C,
    const float *__restrict__ dy, const float *__restrict__ Gws, const float *__restrict__ DTws,
    const float *__restrict__ gh, const Thp *__restrict__ hprev, float *__restrict__ dB,
    float *__restrict__ dC, int64_t T, int32_t H, int32_t G, int32_t nc) {
    constexpr int NB = L / 64, TN = N / 16;
    __shared__ __align__(16) float As[KT * LD];
    __shared__ __align__(16) float Bs[KT * (N + 4)];
    const int64_t blk = blockIdx.x;
    const int orient = (int)(blk & 1);
    const int rb = (int)((blk >> 1) % NB);
    const int64_t bcg = (blk >> 1) / NB;            // (b*nc + c)*G + g
    const int32_t g = (int32_t)(bcg % G);
    const int64_t bc = bcg / G;
    const int32_t c = (int32_t)(bc % nc);
    const int64_t b = bc / nc;
    const int hpg = H / G;
    const int r0 = 64 * rb;
    const int tid = threadIdx.x;
    const int m0 = 4 * (tid >> 4), cj = 4 * (tid & 15), q0n = TN * (tid & 15);
    const int64_t tc = (int64_t)c * L;
    // M(row, col) over the columns of 64-wide blocks; orientation 0: rows k of
    // this block, columns j <= k; orientation 1: rows j of this block, columns k >= j
    float M[NB][4][4] = {};
    float acc2[4][TN] = {};                         // the inter-chunk term, [row][n]
    for (int hh = 0; hh < hpg; ++hh) {
        const int32_t h = g * hpg + hh;
        const int64_t unit = ((b * H) + h) * nc + c;
        const float *Gc = Gws + unit * L, *DTc = DTws + unit * L;
        const float glast = Gc[L - 1];
#pragma unroll
        for (int ob = 0; ob < NB; ++ob) {
            if (orient == 0 ? ob > rb : ob < rb) continue;
            // dYX block: orientation 0 -> dy_rows . x_cols, 1 -> x_rows . dy_cols (K = P)
            float a4[4][4] = {};
            for (int p0 = 0; p0 < P; p0 += KT) {
                __syncthreads();
                for (int e = tid; e < KT * 64; e += 256) {
                    const int r = e / KT, q = e % KT;
                    const int64_t tr = tc + r0 + r, to = tc + 64 * ob + r;
                    const int64_t ir = ((b * T + (tr < T ? tr : 0)) * H + h) * P + p0 + q;
                    const int64_t io = ((b * T + (to < T ? to : 0)) * H + h) * P + p0 + q;
                    const float rv = tr < T ? (orient == 0 ? dy[ir] : ld1(x + ir)) : 0.f;
                    const float ov = to < T ? (orient == 0 ? ld1(x + io) : dy[io]) : 0.f;
                    As[q * LD + r] = rv;
                    Bs[q * LD + r] = ov;
                }
                __syncthreads();
                mm_acc<4, 4>(a4, As, LD, Bs, LD, m0, cj);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = r0 + m0 + i, oo = 64 * ob + cj + j;
                    const int k = orient == 0 ? rr : oo, jx = orient == 0 ? oo : rr;
                    M[ob][i][j] += k >= jx ? fast_exp2(Gc[k] - Gc[jx]) * DTc[jx] * a4[i][j] : 0.f;
                }
        }
        // inter: orientation 0: exp2(G_k) h_prev^T dy_k; 1: dt_j exp2(G_last - G_j) ghat^T x_j
        const float *ghc = gh + unit * (int64_t)(P * N);
        const Thp *hpc = hprev + unit * (int64_t)(P * N);
        for (int p0 = 0; p0 < P; p0 += KT) {
            __syncthreads();
            for (int e = tid; e < KT * 64; e += 256) {
                const int r = e / KT, q = e % KT;
                const int rr = r0 + r;
                const int64_t t = tc + rr;
                const int64_t ix = ((b * T + (t < T ? t : 0)) * H + h) * P + p0 + q;
                float v = 0.f;
                if (t < T)
                    v = orient == 0 ? dy[ix] * fast_exp2(Gc[rr])
                                    : ld1(x + ix) * DTc[rr] * fast_exp2(glast - Gc[rr]);
                As[q * LD + r] = v;
            }
            for (int e = tid; e < KT * N; e += 256) {
                const int q = e / N, n = e % N;
                Bs[q * (N + 4) + n] = orient == 0 ? ld1(hpc + (p0 + q) * N + n)
                                                  : ghc[(p0 + q) * N + n];
            }
            __syncthreads();
            mm_acc<4, TN>(acc2, As, LD, Bs, N + 4, m0, q0n);
        }
    }
    // out(row, n) += sum_col M(row, col) V_col[n], V = B (orientation 0) or C (1)
    for (int ob = 0; ob < NB; ++ob) {
        if (orient == 0 ? ob > rb : ob < rb) continue;
        for (int h0 = 0; h0 < 64; h0 += KT) {
            __syncthreads();
            // this thread's M columns cj..cj+3 that fall in [h0, h0+KT)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = cj + j;
                if (col >= h0 && col < h0 + KT)
#pragma unroll
                    for (int i = 0; i < 4; ++i) As[(col - h0) * LD + m0 + i] = M[ob][i][j];
            }
            for (int e = tid; e < KT * N; e += 256) {
                const int q = e / N, n = e % N;
                const int64_t t = tc + 64 * ob + h0 + q;
                const Tio *V = orient == 0 ? B : C;
                Bs[q * (N + 4) + n] = t < T ? ld1(V + ((b * T + t) * G + g) * N + n) : 0.f;
            }
            __syncthreads();
            mm_acc<4, TN>(acc2, As, LD, Bs, N + 4, m0, q0n);
        }
    }
    float *out = orient == 0 ? dC : dB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = tc + r0 + m0 + i;
        if (t < T)
#pragma unroll
            for (int j = 0; j < TN; j += 4)
                *reinterpret_cast<float4 *>(out + ((b * T + t) * G + g) * N + q0n + j) =
                    make_float4(acc2[i][j], acc2[i][j + 1], acc2[i][j + 2], acc2[i][j + 3]);
    }
}

// ---- bwd_dc_mfma: dC on bf16 MFMA (bf16 io), and M for bwd_db_mfma ---------
// One block of WPB 16-row strips k of one (b, c, g) per workgroup (with two
// blocks per chunk, the outer strips in one and the middle ones in the other,
// which balances their causal tiles), one strip per wavefront: per head, the
// strip's dy rows times the x
// rows of the chunk (decayed and masked into M), and the inter term
// exp2(G) dy h_prev^T; after the heads, M B.  Per head the x rows and h_prev
// (transposed to [n][p]) are staged in LDS; the strip's own rows are the A
// operands, straight from global memory.  v_mfma_f32_16x16x32_bf16 layouts:
// A lane l holds row l%16, k 8(l/16)..+7; B lane l holds column l%16, the same
// k; D lane l holds rows 4(l/16)+e, column l%16.  M stays in the accumulators
// over the heads (fp32), is stored transposed for dB = M^T C, and goes
// through LDS for the final product.
// Precision: dB and dC are small differences of large terms near the end of a
// sequence (where dfinal enters), so every fp32 operand is carried as a bf16
// head plus a bf16 remainder (x, B and C are bf16 already): products of two
// split operands take three MFMAs (hi.hi + hi.lo + lo.hi), of one split
// operand two, which leaves about 2^-16 of relative error instead of 2^-9.

template <int L, int N, int WPB>
__global__ __launch_bounds__(64 * WPB) void bwd_dc_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ B, const float *__restrict__ dy,
    const float *__restrict__ Gws, const float *__restrict__ DTws,
    const float *__restrict__ hprev, float *__restrict__ out, float *__restrict__ MT, int64_t T,
    int32_t H, int32_t G, int32_t nc) {
    constexpr int NT = L / 16, NN = N / 16;
    constexpr int RB = 16 * WPB;                      // rows per workgroup (one strip per wavefront)
    constexpr int NTH = 64 * WPB;
    constexpr int NIB = N > RB ? N : RB;              // Ib rows: n, or the M remainder's rows
    __shared__ __align__(16) uint16_t Cs[L * SP];     // x rows [row][p]; final: M
    __shared__ __align__(16) uint16_t Ib[2][NIB * SP];  // h_prev^T [n][p]; final: B^T
    __shared__ float Gs[L], DTs[L];
    const int64_t blk = xcd_remap(blockIdx.x, gridDim.x);   // row blocks of a group on one XCD
    const int rb = (int)(blk % (L / RB));
    const int64_t bcg = blk / (L / RB);               // (b*nc + c)*G + g
    const int32_t g = (int32_t)(bcg % G);
    const int64_t bc = bcg / G;
    const int32_t c = (int32_t)(bc % nc);
    const int64_t b = bc / nc;
    const int hpg = H / G;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int m = lane & 15, q = lane >> 4;
    // this wavefront's 16-row strip: with two row blocks per chunk, block 0
    // takes the first and the last WPB/2 strips and block 1 the middle ones,
    // so both hold the same number of causal tiles
    constexpr int NSTRIP = L / 16;
    const int strip = (L / RB == 2) ? (rb == 0 ? (w < WPB / 2 ? w : NSTRIP - WPB + w) : WPB / 2 + w) : w;
    const int srow = 16 * strip;
    const int64_t tc = (int64_t)c * L;
    // columns [0, c_hi): on or below the diagonal of the block's last strip
    const int c_hi = (L / RB == 2 && rb == 1) ? 16 * (WPB / 2 + WPB) : L;
    const int arow = srow + m;                        // this lane's A-operand row
    const int64_t ta = tc + arow;
    f32x4 Macc[NT];
    f32x4 dacc[NN];
#pragma unroll
    for (int i = 0; i < NT; ++i) Macc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NN; ++i) dacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // staging items per thread: x rows (8 p each), h_prev (two p rows x 4 n each)
    static_assert(NTH >= L, "one G and DT value per thread");
    constexpr int NCI = (L * (P / 8) + NTH - 1) / NTH;
    constexpr int NII = (P * N / 8 + NTH - 1) / NTH;
    const int ncols = c_hi * (P / 8);
    // every operand of head hh + 1 (x rows, h_prev, G, DT and the strip's dy
    // rows) loads into registers while head hh computes
    uint4 cx[NCI];
    float4 iv[NII][2];
    float gl = 0.f, dl = 0.f;
    float4 ar[2][2];                                  // the strip's own dy rows
    auto load_head = [&](int hh) {
        const int32_t h = g * hpg + hh;
        const int64_t unit = ((b * H) + h) * nc + c;
        if (tid < L) {
            gl = Gws[unit * L + tid];
            dl = DTws[unit * L + tid];
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int64_t o = ((b * T + (ta < T ? ta : 0)) * H + h) * P + 32 * st + 8 * q;
            ar[st][0] = ta < T ? *reinterpret_cast<const float4 *>(dy + o) : make_float4(0.f, 0.f, 0.f, 0.f);
            ar[st][1] = ta < T ? *reinterpret_cast<const float4 *>(dy + o + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < NCI; ++j) {
            const int e = tid + j * NTH;
            const int r = e / (P / 8), p8 = 8 * (e % (P / 8));
            const int64_t t = tc + r;
            const bool ok = e < ncols && t < T;
            const int64_t o = ((b * T + (ok ? t : 0)) * H + h) * P + p8;
            cx[j] = ok ? *reinterpret_cast<const uint4 *>(x + o) : make_uint4(0u, 0u, 0u, 0u);
        }
        const float *src = hprev + unit * (int64_t)(P * N);
#pragma unroll
        for (int j = 0; j < NII; ++j) {
            const int e = tid + j * NTH;
            const int p = 2 * (e % (P / 2)), n4 = 4 * (e / (P / 2));
            const bool ok = e < P * N / 8;
            iv[j][0] = ok ? *reinterpret_cast<const float4 *>(src + p * N + n4) : make_float4(0.f, 0.f, 0.f, 0.f);
            iv[j][1] = ok ? *reinterpret_cast<const float4 *>(src + (p + 1) * N + n4)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    load_head(0);
    for (int hh = 0; hh < hpg; ++hh) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NCI; ++j) {
            const int e = tid + j * NTH;
            if (e < ncols) *reinterpret_cast<uint4 *>(&Cs[(e / (P / 8)) * SP + 8 * (e % (P / 8))]) = cx[j];
        }
        // h_prev transposed to [n][p], as hi + lo: a lane takes rows p, p+1 and
        // writes 32-bit pairs, consecutive lanes consecutive pairs
#pragma unroll
        for (int j = 0; j < NII; ++j) {
            const int e = tid + j * NTH;
            if (e < P * N / 8) {
                const int p = 2 * (e % (P / 2)), n4 = 4 * (e / (P / 2));
                const float a0[4] = {iv[j][0].x, iv[j][0].y, iv[j][0].z, iv[j][0].w};
                const float a1[4] = {iv[j][1].x, iv[j][1].y, iv[j][1].z, iv[j][1].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t hi, lo;
                    split2(a0[i], a1[i], hi, lo);
                    *reinterpret_cast<uint32_t *>(&Ib[0][(n4 + i) * SP + p]) = hi;
                    *reinterpret_cast<uint32_t *>(&Ib[1][(n4 + i) * SP + p]) = lo;
                }
            }
        }
        if (tid < L) {
            Gs[tid] = gl;
            DTs[tid] = dl;
        }
        __syncthreads();
        // A operands: the strip's dy rows (plain, and times exp2(G) for the inter term)
        const float sc = fast_exp2(Gs[arow]);
        // row factors of the off-diagonal decay, against the strip's first row
        const float gedge = Gs[srow];
        float rowf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) rowf[e] = fast_exp2(Gs[srow + 4 * q + e] - gedge);
        bf16x8 aS[2], aSl[2], aI[2], aIl[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const float f[8] = {ar[st][0].x, ar[st][0].y, ar[st][0].z, ar[st][0].w,
                                ar[st][1].x, ar[st][1].y, ar[st][1].z, ar[st][1].w};
            uint4 hi, lo;
            split8(f, hi, lo);
            aS[st] = as_bf16x8(hi);
            aSl[st] = as_bf16x8(lo);
            float fs[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) fs[i] = f[i] * sc;
            split8(fs, hi, lo);
            aI[st] = as_bf16x8(hi);
            aIl[st] = as_bf16x8(lo);
        }
        if (hh + 1 < hpg) load_head(hh + 1);   // gl, dl and ar are consumed
        // S tiles on or below the diagonal, decayed and masked into M
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
            if (16 * jt > srow) continue;             // wholly masked
            f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int off = (16 * jt + m) * SP + 32 * st + 8 * q;
                const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4 *>(&Cs[off]));
                s = mfma16x16x32(aS[st], bh, s);
                s = mfma16x16x32(aSl[st], bh, s);     // dy remainder . x
            }
            const int col = 16 * jt + m;
            const float gc = Gs[col], dc = DTs[col];
            if (16 * jt == srow) {
                // the diagonal tile: the exact pairwise decay, masked
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = srow + 4 * q + e;
                    Macc[jt][e] += row >= col ? fast_exp2(Gs[row] - gc) * dc * s[e] : 0.f;
                }
            } else {
                // below the diagonal every pair counts, and the decay splits at
                // the strip's first row into a row factor and a column factor,
                // both at most 1: one exp2 per tile instead of four
                const float cf = fast_exp2(gedge - gc) * dc;
#pragma unroll
                for (int e = 0; e < 4; ++e) Macc[jt][e] += rowf[e] * (cf * s[e]);
            }
        }
        // inter term: (exp2(G) dy rows) x h_prev, K = P, three products
#pragma unroll
        for (int nt = 0; nt < NN; ++nt)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int off = (16 * nt + m) * SP + 32 * st + 8 * q;
                const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4 *>(&Ib[0][off]));
                const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4 *>(&Ib[1][off]));
                dacc[nt] = mfma16x16x32(aI[st], bh, dacc[nt]);
                dacc[nt] = mfma16x16x32(aI[st], bl, dacc[nt]);
                dacc[nt] = mfma16x16x32(aIl[st], bh, dacc[nt]);
            }
    }
    // M of the strip's rows, all L columns (zero where masked), transposed
    // into MT[col][row] for the dB pass: lane (m, q) holds rows 4q..4q+3 of
    // column 16 jt + m
    {
        float *mt = MT + bcg * (int64_t)(L * L) + srow + 4 * q;
#pragma unroll
        for (int jt = 0; jt < NT; ++jt)
            *reinterpret_cast<float4 *>(mt + (int64_t)(16 * jt + m) * L) =
                make_float4(Macc[jt][0], Macc[jt][1], Macc[jt][2], Macc[jt][3]);
    }
    // final: dC(row, n) += sum_col M(row, col) B_col[n];
    // M goes through LDS as hi (rows 0..RB-1 of Cs) + lo (rows 0..RB-1 of Ib[1])
    for (int cc = 0; cc < c_hi / 64; ++cc) {
        __syncthreads();
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
            if (jt / 4 != cc) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint16_t hi, lo;
                split1(Macc[jt][e], hi, lo);
                const int r = 16 * w + 4 * q + e, cl = 16 * (jt % 4) + m;
                Cs[r * SP + cl] = hi;
                Ib[1][r * SP + cl] = lo;
            }
        }
        // B rows of the chunk, transposed to [n][token]: a lane takes tokens r, r+1
        for (int e = tid; e < 64 * N / 16; e += NTH) {
            const int r = 2 * (e % 32), n8 = 8 * (e / 32);
            const int64_t t = tc + 64 * cc + r;
            uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = v0;
            if (t < T) v0 = *reinterpret_cast<const uint4 *>(B + ((b * T + t) * G + g) * N + n8);
            if (t + 1 < T) v1 = *reinterpret_cast<const uint4 *>(B + ((b * T + t + 1) * G + g) * N + n8);
            const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w}, w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<uint32_t *>(&Ib[0][(n8 + 2 * i) * SP + r]) = pair16(w0[i], w1[i]);
                *reinterpret_cast<uint32_t *>(&Ib[0][(n8 + 2 * i + 1) * SP + r]) =
                    pair16(w0[i] >> 16, w1[i] >> 16);
            }
        }
        __syncthreads();
        bf16x8 aM[2], aMl[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            aM[st] = as_bf16x8(*reinterpret_cast<const uint4 *>(&Cs[(16 * w + m) * SP + 32 * st + 8 * q]));
            aMl[st] = as_bf16x8(
                *reinterpret_cast<const uint4 *>(&Ib[1][(16 * w + m) * SP + 32 * st + 8 * q]));
        }
#pragma unroll
        for (int nt = 0; nt < NN; ++nt)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const bf16x8 bv = as_bf16x8(
                    *reinterpret_cast<const uint4 *>(&Ib[0][(16 * nt + m) * SP + 32 * st + 8 * q]));
                dacc[nt] = mfma16x16x32(aM[st], bv, dacc[nt]);
                dacc[nt] = mfma16x16x32(aMl[st], bv, dacc[nt]);
            }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t t = tc + srow + 4 * q + e;
        if (t < T)
#pragma unroll
            for (int nt = 0; nt < NN; ++nt)
                out[((b * T + t) * G + g) * N + 16 * nt + m] = dacc[nt][e];
    }
}

// ---- bwd_db_mfma: dB rows j of one (b, chunk, group) from the M that
// bwd_dc_mfma stored (transposed, fp32):
//   dB(j, n) = sum_{k >= j} M(k, j) C_k[n] + sum_h dt_j exp2(G_last - G_j) x_j . ghat_h[:, n]
// Per head only ghat (staged transposed as hi + lo) and the strip's x rows
// (A operands from global memory) are read; M^T rows come from global memory
// as hi + lo A operands for the final product with C (staged transposed).
template <int L, int N, int WPB>
__global__ __launch_bounds__(64 * WPB) void bwd_db_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ C, const float *__restrict__ Gws,
    const float *__restrict__ DTws, const float *__restrict__ gh, const float *__restrict__ MT,
    float *__restrict__ out, int64_t T, int32_t H, int32_t G, int32_t nc) {
    constexpr int NN = N / 16;
    constexpr int RB = 16 * WPB;
    constexpr int NTH = 64 * WPB;
    __shared__ __align__(16) uint16_t Ib[2][N * SP];  // ghat^T [n][p] hi + lo; final: C^T
    const int64_t blk = xcd_remap(blockIdx.x, gridDim.x);
    const int rb = (int)(blk % (L / RB));
    const int64_t bcg = blk / (L / RB);               // (b*nc + c)*G + g
    const int32_t g = (int32_t)(bcg % G);
    const int64_t bc = bcg / G;
    const int32_t c = (int32_t)(bc % nc);
    const int64_t b = bc / nc;
    const int hpg = H / G;
    const int r0 = RB * rb;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int m = lane & 15, q = lane >> 4;
    const int64_t tc = (int64_t)c * L;
    const int arow = r0 + 16 * w + m;                 // this lane's A-operand row
    const int64_t ta = tc + arow;
    f32x4 dacc[NN];
#pragma unroll
    for (int i = 0; i < NN; ++i) dacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int NII = (P * N / 8 + NTH - 1) / NTH;
    // one head ahead: ghat, the strip row's G, DT and x of head hh + 1 load
    // into registers while head hh computes
    float4 iv[NII][2];
    float ga = 0.f, glast = 0.f, da = 0.f;
    uint4 ar[2];
    auto load_head = [&](int hh) {
        const int32_t h = g * hpg + hh;
        const int64_t unit = ((b * H) + h) * nc + c;
        const float *src = gh + unit * (int64_t)(P * N);
#pragma unroll
        for (int j = 0; j < NII; ++j) {
            const int e = tid + j * NTH;
            const int p = 2 * (e % (P / 2)), n4 = 4 * (e / (P / 2));
            const bool ok = e < P * N / 8;
            iv[j][0] = ok ? *reinterpret_cast<const float4 *>(src + p * N + n4) : make_float4(0.f, 0.f, 0.f, 0.f);
            iv[j][1] = ok ? *reinterpret_cast<const float4 *>(src + (p + 1) * N + n4)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        ga = Gws[unit * L + arow];
        glast = Gws[unit * L + L - 1];
        da = DTws[unit * L + arow];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int64_t o = ((b * T + (ta < T ? ta : 0)) * H + h) * P + 32 * st + 8 * q;
            ar[st] = ta < T ? *reinterpret_cast<const uint4 *>(x + o) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    load_head(0);
    for (int hh = 0; hh < hpg; ++hh) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NII; ++j) {
            const int e = tid + j * NTH;
            if (e < P * N / 8) {
                const int p = 2 * (e % (P / 2)), n4 = 4 * (e / (P / 2));
                const float a0[4] = {iv[j][0].x, iv[j][0].y, iv[j][0].z, iv[j][0].w};
                const float a1[4] = {iv[j][1].x, iv[j][1].y, iv[j][1].z, iv[j][1].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t hi, lo;
                    split2(a0[i], a1[i], hi, lo);
                    *reinterpret_cast<uint32_t *>(&Ib[0][(n4 + i) * SP + p]) = hi;
                    *reinterpret_cast<uint32_t *>(&Ib[1][(n4 + i) * SP + p]) = lo;
                }
            }
        }
        // A operand: the strip's x rows times dt exp2(G_last - G), hi + lo
        const float sc = da * fast_exp2(glast - ga);
        bf16x8 aI[2], aIl[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const uint4 u = ar[st];
            const float fs[8] = {bf16_lo(u.x) * sc, bf16_hi(u.x) * sc, bf16_lo(u.y) * sc,
                                 bf16_hi(u.y) * sc, bf16_lo(u.z) * sc, bf16_hi(u.z) * sc,
                                 bf16_lo(u.w) * sc, bf16_hi(u.w) * sc};
            uint4 hi, lo;
            split8(fs, hi, lo);
            aI[st] = as_bf16x8(hi);
            aIl[st] = as_bf16x8(lo);
        }
        if (hh + 1 < hpg) load_head(hh + 1);
        __syncthreads();
#pragma unroll
        for (int nt = 0; nt < NN; ++nt)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int off = (16 * nt + m) * SP + 32 * st + 8 * q;
                const bf16x8 bh = as_bf16x8(*reinterpret_cast<const uint4 *>(&Ib[0][off]));
                const bf16x8 bl = as_bf16x8(*reinterpret_cast<const uint4 *>(&Ib[1][off]));
                dacc[nt] = mfma16x16x32(aI[st], bh, dacc[nt]);
                dacc[nt] = mfma16x16x32(aI[st], bl, dacc[nt]);
                dacc[nt] = mfma16x16x32(aIl[st], bh, dacc[nt]);
            }
    }
    // final: dB(j, n) += sum_k M^T(j, k) C_k[n] over k >= r0 (M is zero above
    // its diagonal), 64 tokens k at a time
    const float *mrow = MT + bcg * (int64_t)(L * L) + (int64_t)arow * L;
    for (int cc = r0 / 64; cc < L / 64; ++cc) {
        float4 mv[2][2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            mv[st][0] = *reinterpret_cast<const float4 *>(mrow + 64 * cc + 32 * st + 8 * q);
            mv[st][1] = *reinterpret_cast<const float4 *>(mrow + 64 * cc + 32 * st + 8 * q + 4);
        }
        __syncthreads();
        // C rows of the chunk, transposed to [n][token]: a lane takes tokens r, r+1
        for (int e = tid; e < 64 * N / 16; e += NTH) {
            const int r = 2 * (e % 32), n8 = 8 * (e / 32);
            const int64_t t = tc + 64 * cc + r;
            uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = v0;
            if (t < T) v0 = *reinterpret_cast<const uint4 *>(C + ((b * T + t) * G + g) * N + n8);
            if (t + 1 < T) v1 = *reinterpret_cast<const uint4 *>(C + ((b * T + t + 1) * G + g) * N + n8);
            const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w}, w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<uint32_t *>(&Ib[0][(n8 + 2 * i) * SP + r]) = pair16(w0[i], w1[i]);
                *reinterpret_cast<uint32_t *>(&Ib[0][(n8 + 2 * i + 1) * SP + r]) =
                    pair16(w0[i] >> 16, w1[i] >> 16);
            }
        }
        __syncthreads();
        bf16x8 aM[2], aMl[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const float f[8] = {mv[st][0].x, mv[st][0].y, mv[st][0].z, mv[st][0].w,
                                mv[st][1].x, mv[st][1].y, mv[st][1].z, mv[st][1].w};
            uint4 hi, lo;
            split8(f, hi, lo);
            aM[st] = as_bf16x8(hi);
            aMl[st] = as_bf16x8(lo);
        }
#pragma unroll
        for (int nt = 0; nt < NN; ++nt)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const bf16x8 bv = as_bf16x8(
                    *reinterpret_cast<const uint4 *>(&Ib[0][(16 * nt + m) * SP + 32 * st + 8 * q]));
                dacc[nt] = mfma16x16x32(aM[st], bv, dacc[nt]);
                dacc[nt] = mfma16x16x32(aMl[st], bv, dacc[nt]);
            }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t t = tc + r0 + 16 * w + 4 * q + e;
        if (t < T)
#pragma unroll
            for (int nt = 0; nt < NN; ++nt)
                out[((b * T + t) * G + g) * N + 16 * nt + m] = dacc[nt][e];
    }
}

// ---- bwd_dx_mfma: bwd_dx on bf16 MFMA with split operands (bf16 io) ------
// One (b, c, h) per workgroup of L/16 wavefronts, wavefront w owning rows
// 16w .. 16w+15, so each head's operands are staged once and the causal work
// per wavefront is the same (U takes k >= i, Y takes j <= i); MFMA layouts
// as for bwd_dc_mfma.  Products (K in brackets):
//   U_intra(i, p) = sum_{k >= i} W(k, i) dy_k[p]    [k]  W(k, i) = exp2(G_k - G_i) CB(k, i)
//   Y_intra(i, p) = sum_{j <= i} V(i, j) x_j[p]     [j]  V(i, j) = exp2(G_i - G_j) CB(i, j) dt_j
//   U_inter(i, p) = sum_n B_i[n] ghat[p][n]         [n]
//   Y_inter(i, p) = sum_n C_i[n] h_prev[p][n]       [n]
// the inter products scaled per row afterwards (exp2(G_last - G_i), exp2(G_i)).
// K runs in 32-token steps.  A step wholly on the causal side of a strip
// splits the decay at the step's edge token e (the first for U, the last for
// Y) into a token factor and a row factor, both at most 1:
//   exp2(G_k - G_i) = exp2(G_k - G_e) exp2(G_e - G_i),
// so its A operand is C B^T itself (head-independent, split into three bf16
// terms once per group), its B operand the staged dy or dt x scaled by the
// token factor, and the row factor scales the step's product.  The step that
// holds the strip's rows takes the exact pairwise decay per element.  These
// sums feed ddt and the decay gradients, so every fp32 operand is carried as
// three bf16 terms (two terms left the full-size dA at 0.7 of its bar) and a
// product takes the six MFMAs of order 2^-16 and above.
template <int L, int N>
__global__ __launch_bounds__(4 * L) void bwd_dx_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ B, const uint16_t *__restrict__ C,
    const float *__restrict__ D, const float *__restrict__ dy, const float *__restrict__ Gws,
    const float *__restrict__ DTws, const uint16_t *__restrict__ CB3, const uint16_t *__restrict__ CBT3, int64_t plane,
    const float *__restrict__ gh, const float *__restrict__ hprev, float *__restrict__ dx,
    float *__restrict__ tok, int64_t T, int32_t H, int32_t G, int32_t nc, int64_t ntok) {
    constexpr int NB = L / 64, NP = P / 16, PN = N + 16;   // PN: 72- or 40-word rows, conflict-free
    // the chunk tiles keep a 36-word pitch: their read conflicts cost no measurable time
    // here, and the conflict-free 40-word pitch makes the allocator spill
    constexpr int SPX = P + 8;
    constexpr int NTH = 4 * L;                        // L/16 wavefronts: one 16-row strip each
    // phases: U and Y over token chunk 0..NB-1 (chunk ck holds steps 2ck and
    // 2ck+1; U takes the steps at or after a strip's own, Y those at or
    // before it, so every wavefront has two or three steps in each phase),
    // then the ghat and the h_prev inter products.  Each phase's staged
    // operands are loaded into registers while the previous phase computes
    // (one workgroup fills a CU).
    constexpr int NPH = NB + 2;
    // staging items of a chunk phase: (token pair, 4 p) of dy, then
    // (token pair, 8 p) of x; of an inter phase: 4 consecutive [p][n] values
    constexpr int N_DY = 64 * (P / 8), N_X = 64 * (P / 16), N_S = N_DY + N_X, N_I = P * N / 4;
    constexpr int IT_S = (N_S + NTH - 1) / NTH, IT_I = (N_I + NTH - 1) / NTH;
    constexpr int NSR = 2 * IT_S > IT_I ? 2 * IT_S : IT_I;
    // phase-shared LDS, [p][64 tokens] tiles: tiles 0..2 hold dy in three
    // terms, 3..5 dy times its token factor, 6 x, 7..9 dt x times its token
    // factor; the inter phases use Ih/Im/Il [p][N]
    constexpr int TY = 6;                             // first Y tile
    constexpr int NLDS = 3 * P * PN > 10 * P * SPX ? 3 * P * PN : 10 * P * SPX;
    __shared__ __align__(16) uint16_t lds[NLDS];
    __shared__ float Gs[L], DTs[L];
    uint16_t *const Tu = lds;
    uint16_t *const Ih = lds, *const Im = lds + P * PN, *const Il = lds + 2 * P * PN;
    // logical block order (b, c, g, head) with the head fastest and
    // consecutive ids on one XCD: the heads of a group reuse the same C B^T
    // rows from that XCD's L2
    const int64_t blk = xcd_remap(blockIdx.x, gridDim.x);
    const int hpg = H / G;
    const int32_t hh = (int32_t)(blk % hpg);
    const int64_t bcg = blk / hpg;                    // (b*nc + c)*G + g
    const int32_t g = (int32_t)(bcg % G);
    const int64_t bc = bcg / G;
    const int32_t c = (int32_t)(bc % nc);
    const int64_t b = bc / nc;
    const int32_t h = g * hpg + hh;
    const int64_t bh = b * H + h;
    const int64_t unit = bh * nc + c;                 // (b*H + h)*nc + c
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int m = lane & 15, q = lane >> 4;
    const int64_t tc = (int64_t)c * L;
    const int arow = 16 * w + m;                      // A-operand row of this lane
    const int sdiag = w >> 1;                         // the 32-token step holding the strip
    const int64_t ta = tc + arow;
    const int64_t rowoff = bcg * (int64_t)(L * L) + (int64_t)arow * L;
    for (int e = tid; e < L; e += NTH) {
        Gs[e] = Gws[unit * L + e];
        DTs[e] = DTws[unit * L + e];
    }
    f32x4 U[NP], Y[NP], Ui[NP], Yi[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        U[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        Y[i] = U[i];
    }
    uint4 sr[NSR];            // staging registers of the next phase
    uint4 ra[N / 32];         // this lane's B or C row of the next inter phase

    auto load_phase = [&](int ph) {
        if (ph < NB) {
#pragma unroll
            for (int j = 0; j < IT_S; ++j) {
                const int e = tid + j * NTH;
                sr[2 * j] = make_uint4(0u, 0u, 0u, 0u);
                sr[2 * j + 1] = sr[2 * j];
                if (e < N_DY) {
                    const int r = 2 * (e % 32), pc = 4 * (e / 32);
                    const int64_t t = tc + 64 * ph + r;
                    if (t < T)
                        sr[2 * j] = *reinterpret_cast<const uint4 *>(dy + ((b * T + t) * H + h) * P + pc);
                    if (t + 1 < T)
                        sr[2 * j + 1] =
                            *reinterpret_cast<const uint4 *>(dy + ((b * T + t + 1) * H + h) * P + pc);
                } else if (e < N_S) {
                    const int ex = e - N_DY;
                    const int r = 2 * (ex % 32), pc = 8 * (ex / 32);
                    const int64_t t = tc + 64 * ph + r;
                    if (t < T)
                        sr[2 * j] = *reinterpret_cast<const uint4 *>(x + ((b * T + t) * H + h) * P + pc);
                    if (t + 1 < T)
                        sr[2 * j + 1] =
                            *reinterpret_cast<const uint4 *>(x + ((b * T + t + 1) * H + h) * P + pc);
                }
            }
        } else {
            const float *src = (ph == NB ? gh : hprev) + unit * (int64_t)(P * N);
#pragma unroll
            for (int j = 0; j < NSR; ++j) {
                const int e = tid + j * NTH;
                sr[j] = make_uint4(0u, 0u, 0u, 0u);
                if (j < IT_I && e < N_I) {
                    const int pp = e / (N / 4), n4 = 4 * (e % (N / 4));
                    sr[j] = *reinterpret_cast<const uint4 *>(src + pp * N + n4);
                }
            }
            const uint16_t *rows = (ph == NB ? B : C) + ((b * T + (ta < T ? ta : 0)) * G + g) * N;
#pragma unroll
            for (int ks = 0; ks < N / 32; ++ks)
                ra[ks] = ta < T ? *reinterpret_cast<const uint4 *>(rows + 32 * ks + 8 * q)
                                : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_phase = [&](int ph) {
        if (ph < NB) {
#pragma unroll
            for (int j = 0; j < IT_S; ++j) {
                const int e = tid + j * NTH;
                if (e < N_DY) {                        // dy, and dy times its token factor
                    const int r = 2 * (e % 32), p4 = 4 * (e / 32);
                    const int k = 64 * ph + r;         // tokens k, k+1 (one 32-token step)
                    const float ge = Gs[k & ~31];
                    const float f0 = fast_exp2(Gs[k] - ge), f1 = fast_exp2(Gs[k + 1] - ge);
                    const uint4 u0 = sr[2 * j], u1 = sr[2 * j + 1];
                    const float a0[4] = {__uint_as_float(u0.x), __uint_as_float(u0.y),
                                         __uint_as_float(u0.z), __uint_as_float(u0.w)};
                    const float a1[4] = {__uint_as_float(u1.x), __uint_as_float(u1.y),
                                         __uint_as_float(u1.z), __uint_as_float(u1.w)};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t s0, s1, s2;
                        const int o = (p4 + i) * SPX + r;
                        split2x3(a0[i], a1[i], s0, s1, s2);
                        *reinterpret_cast<uint32_t *>(Tu + o) = s0;
                        *reinterpret_cast<uint32_t *>(Tu + P * SPX + o) = s1;
                        *reinterpret_cast<uint32_t *>(Tu + 2 * P * SPX + o) = s2;
                        split2x3(a0[i] * f0, a1[i] * f1, s0, s1, s2);
                        *reinterpret_cast<uint32_t *>(Tu + 3 * P * SPX + o) = s0;
                        *reinterpret_cast<uint32_t *>(Tu + 4 * P * SPX + o) = s1;
                        *reinterpret_cast<uint32_t *>(Tu + 5 * P * SPX + o) = s2;
                    }
                } else if (e < N_S) {                  // x (exact), and dt x times its token factor
                    const int ex = e - N_DY;
                    const int r = 2 * (ex % 32), p8 = 8 * (ex / 32);
                    const int jt = 64 * ph + r;
                    const float ge = Gs[jt | 31];
                    const float f0 = fast_exp2(ge - Gs[jt]) * DTs[jt];
                    const float f1 = fast_exp2(ge - Gs[jt + 1]) * DTs[jt + 1];
                    const uint32_t w0[4] = {sr[2 * j].x, sr[2 * j].y, sr[2 * j].z, sr[2 * j].w};
                    const uint32_t w1[4] = {sr[2 * j + 1].x, sr[2 * j + 1].y, sr[2 * j + 1].z,
                                            sr[2 * j + 1].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const int o = (p8 + 2 * i + hf) * SPX + r;
                            const uint32_t b0 = hf ? w0[i] >> 16 : w0[i] & 0xffffu;
                            const uint32_t b1 = hf ? w1[i] >> 16 : w1[i] & 0xffffu;
                            *reinterpret_cast<uint32_t *>(Tu + TY * P * SPX + o) = pair16(b0, b1);
                            uint32_t s0, s1, s2;
                            split2x3(__uint_as_float(b0 << 16) * f0, __uint_as_float(b1 << 16) * f1, s0,
                                     s1, s2);
                            *reinterpret_cast<uint32_t *>(Tu + (TY + 1) * P * SPX + o) = s0;
                            *reinterpret_cast<uint32_t *>(Tu + (TY + 2) * P * SPX + o) = s1;
                            *reinterpret_cast<uint32_t *>(Tu + (TY + 3) * P * SPX + o) = s2;
                        }
                    }
                }
            }
        } else {                                       // [p][n], three terms
#pragma unroll
            for (int j = 0; j < NSR; ++j) {
                const int e = tid + j * NTH;
                if (j < IT_I && e < N_I) {
                    const int pp = e / (N / 4), n4 = 4 * (e % (N / 4));
                    uint32_t s0a, s1a, s2a, s0b, s1b, s2b;
                    split2x3(__uint_as_float(sr[j].x), __uint_as_float(sr[j].y), s0a, s1a, s2a);
                    split2x3(__uint_as_float(sr[j].z), __uint_as_float(sr[j].w), s0b, s1b, s2b);
                    const int o = pp * PN + n4;
                    *reinterpret_cast<uint2 *>(Ih + o) = make_uint2(s0a, s0b);
                    *reinterpret_cast<uint2 *>(Im + o) = make_uint2(s1a, s1b);
                    *reinterpret_cast<uint2 *>(Il + o) = make_uint2(s2a, s2b);
                }
            }
        }
    };
    // six products of two three-term operands, smallest first
    auto mfma6 = [](const bf16x8 (&a)[3], const bf16x8 (&bb)[3], f32x4 acc) {
        acc = mfma16x16x32(a[2], bb[0], acc);
        acc = mfma16x16x32(a[0], bb[2], acc);
        acc = mfma16x16x32(a[1], bb[1], acc);
        acc = mfma16x16x32(a[1], bb[0], acc);
        acc = mfma16x16x32(a[0], bb[1], acc);
        return mfma16x16x32(a[0], bb[0], acc);
    };
    // one 32-token step s of U (isU) or Y whose staged tokens sit at toff
    auto step = [&](const bool isU, const int s, const int toff, const float g_i) {
        const int k0 = 32 * s + 8 * q;                 // this lane's 8 tokens of it
        if (s == sdiag) {
            // the exact pairwise decay, masked, on C B^T rebuilt in fp32 from
            // its three bf16 terms (their sum is the fp32 value exactly)
            const uint16_t *rowp = (isU ? CBT3 : CB3) + rowoff + k0;
            const uint4 t0 = *reinterpret_cast<const uint4 *>(rowp);
            const uint4 t1 = *reinterpret_cast<const uint4 *>(rowp + plane);
            const uint4 t2 = *reinterpret_cast<const uint4 *>(rowp + 2 * plane);
            const uint32_t w0[4] = {t0.x, t0.y, t0.z, t0.w}, w1[4] = {t1.x, t1.y, t1.z, t1.w},
                           w2[4] = {t2.x, t2.y, t2.z, t2.w};
            float cv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cv[2 * i] = (bf16_lo(w0[i]) + bf16_lo(w1[i])) + bf16_lo(w2[i]);
                cv[2 * i + 1] = (bf16_hi(w0[i]) + bf16_hi(w1[i])) + bf16_hi(w2[i]);
            }
            float av[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = k0 + i;
                av[i] = isU ? (k >= arow ? fast_exp2(Gs[k] - g_i) * cv[i] : 0.f)
                            : (k <= arow ? fast_exp2(g_i - Gs[k]) * cv[i] * DTs[k] : 0.f);
            }
            uint4 a0, a1, a2;
            split8x3(av, a0, a1, a2);
            const bf16x8 a[3] = {as_bf16x8(a0), as_bf16x8(a1), as_bf16x8(a2)};
#pragma unroll
            for (int pt = 0; pt < NP; ++pt) {
                const int off = (16 * pt + m) * SPX + toff;
                if (isU) {
                    const bf16x8 bb[3] = {as_bf16x8(*reinterpret_cast<const uint4 *>(Tu + off)),
                                          as_bf16x8(*reinterpret_cast<const uint4 *>(Tu + P * SPX + off)),
                                          as_bf16x8(*reinterpret_cast<const uint4 *>(Tu + 2 * P * SPX + off))};
                    U[pt] = mfma6(a, bb, U[pt]);
                } else {
                    const bf16x8 bx = as_bf16x8(*reinterpret_cast<const uint4 *>(Tu + TY * P * SPX + off));
                    Y[pt] = mfma16x16x32(a[2], bx, Y[pt]);
                    Y[pt] = mfma16x16x32(a[1], bx, Y[pt]);
                    Y[pt] = mfma16x16x32(a[0], bx, Y[pt]);
                }
            }
        } else if (isU ? s > sdiag : s < sdiag) {
            // wholly causal: C B^T in three terms times the scaled operand
            const uint16_t *rowp = (isU ? CBT3 : CB3) + rowoff + k0;
            const bf16x8 a[3] = {as_bf16x8(*reinterpret_cast<const uint4 *>(rowp)),
                                 as_bf16x8(*reinterpret_cast<const uint4 *>(rowp + plane)),
                                 as_bf16x8(*reinterpret_cast<const uint4 *>(rowp + 2 * plane))};
            const int tb = isU ? 3 : TY + 1;           // first tile of the scaled operand
            f32x4 part[NP];
#pragma unroll
            for (int pt = 0; pt < NP; ++pt) {
                const int off = (16 * pt + m) * SPX + toff;
                const bf16x8 bb[3] = {
                    as_bf16x8(*reinterpret_cast<const uint4 *>(Tu + tb * P * SPX + off)),
                    as_bf16x8(*reinterpret_cast<const uint4 *>(Tu + (tb + 1) * P * SPX + off)),
                    as_bf16x8(*reinterpret_cast<const uint4 *>(Tu + (tb + 2) * P * SPX + off))};
                part[pt] = mfma6(a, bb, f32x4{0.f, 0.f, 0.f, 0.f});
            }
            // the row factor: exp2(G_e - G_i) for U (e the step's first
            // token), exp2(G_i - G_e) for Y (e its last)
            const float ge = Gs[isU ? 32 * s : 32 * s + 31];
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const float gr = Gs[16 * w + 4 * q + e4];
                const float rf = isU ? fast_exp2(ge - gr) : fast_exp2(gr - ge);
#pragma unroll
                for (int pt = 0; pt < NP; ++pt) {
                    if (isU)
                        U[pt][e4] = fmaf(rf, part[pt][e4], U[pt][e4]);
                    else
                        Y[pt][e4] = fmaf(rf, part[pt][e4], Y[pt][e4]);
                }
            }
        }
    };

    // the epilogue's dy (rows i = 16w + 4q + e, columns p = 16 pt + m),
    // loaded during the last phase where the registers allow (at N = 64 the
    // allocator spills with them live; there the epilogue loads them itself)
    constexpr bool kEpiPrefetch = N >= 128;
    float edy[4][NP];
    // dy, x and dx of this (b, c, h) through buffers whose range ends at the
    // sequence end: rows past it read 0 and drop their stores without a
    // branch, so all of a lane's epilogue loads go out before any is used
    const int64_t tok0 = ((b * T + tc) * H + h) * P;
    const uint32_t nvt = (uint32_t)(T - tc < L ? T - tc : L), hpb = (uint32_t)(H * P);
    const auto rdy = make_rsrc(dy + tok0, nvt * hpb * 4u);
    const auto rxx = make_rsrc(x + tok0, nvt * hpb * 2u);
    const auto rdx = make_rsrc(dx + tok0, nvt * hpb * 4u);
    auto eo = [&](int e, int pt) {
        return (uint32_t)(16 * w + 4 * q + e) * hpb + (uint32_t)(16 * pt + m);
    };
    auto load_epilogue = [&]() {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int pt = 0; pt < NP; ++pt)
                edy[e][pt] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdy, 4u * eo(e, pt), 0, 0));
    };

    __syncthreads();
    const float g_i = Gs[arow];
    load_phase(0);
    // unrolled: each phase's code is specialised, so only its registers are live
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
        if (ph == NB)
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                Ui[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                Yi[i] = Ui[i];
            }
        __syncthreads();                               // the previous phase is done with the LDS
        store_phase(ph);
        uint4 rcur[N / 32];
#pragma unroll
        for (int ks = 0; ks < N / 32; ++ks) rcur[ks] = ra[ks];
        if (ph + 1 < NPH) load_phase(ph + 1);
        else if constexpr (kEpiPrefetch) load_epilogue();
        __syncthreads();
        if (ph < NB) {
#pragma unroll
            for (int st = 0; st < 2; ++st) step(true, 2 * ph + st, 32 * st + 8 * q, g_i);
#pragma unroll
            for (int st = 0; st < 2; ++st) step(false, 2 * ph + st, 32 * st + 8 * q, g_i);
        } else {                                       // inter: (B or C rows) x (ghat or h_prev)
            const bool first = ph == NB;
#pragma unroll
            for (int ks = 0; ks < N / 32; ++ks)
#pragma unroll
                for (int pt = 0; pt < NP; ++pt) {
                    const int off = (16 * pt + m) * PN + 32 * ks + 8 * q;
                    const bf16x8 b0 = as_bf16x8(*reinterpret_cast<const uint4 *>(Ih + off));
                    const bf16x8 b1 = as_bf16x8(*reinterpret_cast<const uint4 *>(Im + off));
                    const bf16x8 b2 = as_bf16x8(*reinterpret_cast<const uint4 *>(Il + off));
                    f32x4 acc = first ? Ui[pt] : Yi[pt];
                    acc = mfma16x16x32(as_bf16x8(rcur[ks]), b2, acc);
                    acc = mfma16x16x32(as_bf16x8(rcur[ks]), b1, acc);
                    acc = mfma16x16x32(as_bf16x8(rcur[ks]), b0, acc);
                    if (first)
                        Ui[pt] = acc;
                    else
                        Yi[pt] = acc;
                }
        }
    }
    // ---- epilogue: rows i = 16w + 4q + e, columns p = 16 pt + m
    const float Dh = D[h], glast = Gs[L - 1];
    if constexpr (!kEpiPrefetch) load_epilogue();
    uint32_t xr[4][NP];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int pt = 0; pt < NP; ++pt)
            xr[e][pt] = __builtin_amdgcn_raw_buffer_load_b16(rxx, 2u * eo(e, pt), 0, 0);
    float rowv[3][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * q + e;
        const float su = fast_exp2(glast - Gs[i]), sy = fast_exp2(Gs[i]), dti = DTs[i];
        float xu = 0.f, dyy = 0.f, dyx = 0.f;
#pragma unroll
        for (int pt = 0; pt < NP; ++pt) {
            const float dyv = edy[e][pt];
            const float xv = bf16_to_f32((uint16_t)xr[e][pt]);
            const float u = U[pt][e] + su * Ui[pt][e];
            const float yv = Y[pt][e] + sy * Yi[pt][e];
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Dh * dyv + dti * u), rdx,
                                                  4u * eo(e, pt), 0, 0);
            xu = fmaf(xv, u, xu);
            dyy = fmaf(dyv, yv, dyy);
            dyx = fmaf(dyv, xv, dyx);
        }
        xu = group_sum<16>(xu);                       // over the 16 lanes of one q
        dyy = group_sum<16>(dyy);
        dyx = group_sum<16>(dyx);
        rowv[0][e] = xu;
        rowv[1][e] = dyy - dti * xu;
        rowv[2][e] = dyx;
    }
    // lane m < 4 stores row e = m of each plane; the others aim past the
    // buffer's range and are dropped
    const uint32_t to = m < 4 ? (uint32_t)(16 * w + 4 * q + m) * 4u : 0x7fffffffu;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const float v = m == 0 ? rowv[k][0] : m == 1 ? rowv[k][1] : m == 2 ? rowv[k][2] : rowv[k][3];
        const auto rt = make_rsrc(tok + k * ntok + unit * (int64_t)L, L * 4u);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rt, to, 0, 0);
    }
}

// ---- bwd_dstate_mfma: bwd_dstate on bf16 MFMA (bf16 io) ---------------------
// dSp[p][n] = sum_k exp2(G_k) dy_k[p] C_k[n] for one (b, h, c) per workgroup;
// wavefront w owns rows p = 16w..16w+15 and all N columns.  Both operands
// have K = token, so each 64-token chunk is staged transposed into LDS with
// 32-bit pair writes: (exp2(G) dy)^T in three bf16 terms (the adjoint it
// feeds reaches dx, ddt and dA) and C^T (bf16 already).  Three MFMAs per
// step; layouts as for bwd_dc_mfma.
template <int L, int N>
__global__ __launch_bounds__(256) void bwd_dstate_mfma_kernel(const float *__restrict__ dy,
                                                              const uint16_t *__restrict__ C,
                                                              const float *__restrict__ Gws,
                                                              float *__restrict__ dS, int64_t T,
                                                              int32_t H, int32_t G, int32_t nc) {
    constexpr int NN = N / 16;
    __shared__ __align__(16) uint16_t Dt[3][P * SP];   // (exp2(G) dy)^T, three terms [p][token]
    __shared__ __align__(16) uint16_t Ct[N * SP];      // C^T [n][token]
    __shared__ float Gs[L];
    const int64_t blk = xcd_remap(blockIdx.x, gridDim.x);
    const int hpg = H / G;
    const int32_t h = (int32_t)((blk / hpg) % G) * hpg + (int32_t)(blk % hpg);
    const int32_t g = h / hpg;
    const int32_t c = (int32_t)((blk / H) % nc);
    const int64_t b = blk / H / nc;
    const int64_t unit = (b * H + h) * nc + c;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int m = lane & 15, q = lane >> 4;
    const int64_t tc = (int64_t)c * L;
    for (int e = tid; e < L; e += 256) Gs[e] = Gws[unit * L + e];
    f32x4 acc[NN];
#pragma unroll
    for (int i = 0; i < NN; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kc = 0; kc < L / 64; ++kc) {
        __syncthreads();
        for (int e = tid; e < 64 * (P / 8); e += 256) {       // tokens r, r+1; p4..p4+3
            const int r = 2 * (e % 32), p4 = 4 * (e / 32);
            const int64_t t = tc + 64 * kc + r;
            float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
            if (t < T) v0 = *reinterpret_cast<const float4 *>(dy + ((b * T + t) * H + h) * P + p4);
            if (t + 1 < T)
                v1 = *reinterpret_cast<const float4 *>(dy + ((b * T + t + 1) * H + h) * P + p4);
            const float s0 = fast_exp2(Gs[64 * kc + r]), s1 = fast_exp2(Gs[64 * kc + r + 1]);
            const float a0[4] = {v0.x * s0, v0.y * s0, v0.z * s0, v0.w * s0};
            const float a1[4] = {v1.x * s1, v1.y * s1, v1.z * s1, v1.w * s1};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t w0, w1, w2;
                split2x3(a0[i], a1[i], w0, w1, w2);
                const int o = (p4 + i) * SP + r;
                *reinterpret_cast<uint32_t *>(&Dt[0][o]) = w0;
                *reinterpret_cast<uint32_t *>(&Dt[1][o]) = w1;
                *reinterpret_cast<uint32_t *>(&Dt[2][o]) = w2;
            }
        }
        for (int e = tid; e < 64 * (N / 16); e += 256) {      // tokens r, r+1; n8..n8+7
            const int r = 2 * (e % 32), n8 = 8 * (e / 32);
            const int64_t t = tc + 64 * kc + r;
            uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = v0;
            if (t < T) v0 = *reinterpret_cast<const uint4 *>(C + ((b * T + t) * G + g) * N + n8);
            if (t + 1 < T) v1 = *reinterpret_cast<const uint4 *>(C + ((b * T + t + 1) * G + g) * N + n8);
            const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w}, w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<uint32_t *>(&Ct[(n8 + 2 * i) * SP + r]) = pair16(w0[i], w1[i]);
                *reinterpret_cast<uint32_t *>(&Ct[(n8 + 2 * i + 1) * SP + r]) =
                    pair16(w0[i] >> 16, w1[i] >> 16);
            }
        }
        __syncthreads();
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int ao = (16 * w + m) * SP + 32 * st + 8 * q;
            const bf16x8 a0 = as_bf16x8(*reinterpret_cast<const uint4 *>(&Dt[0][ao]));
            const bf16x8 a1 = as_bf16x8(*reinterpret_cast<const uint4 *>(&Dt[1][ao]));
            const bf16x8 a2 = as_bf16x8(*reinterpret_cast<const uint4 *>(&Dt[2][ao]));
#pragma unroll
            for (int nt = 0; nt < NN; ++nt) {
                const bf16x8 bv = as_bf16x8(
                    *reinterpret_cast<const uint4 *>(&Ct[(16 * nt + m) * SP + 32 * st + 8 * q]));
                acc[nt] = mfma16x16x32(a2, bv, acc[nt]);
                acc[nt] = mfma16x16x32(a1, bv, acc[nt]);
                acc[nt] = mfma16x16x32(a0, bv, acc[nt]);
            }
        }
    }
    float *o = dS + unit * (int64_t)(P * N);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int nt = 0; nt < NN; ++nt) o[(16 * w + 4 * q + e) * N + 16 * nt + m] = acc[nt][e];
}

// ---- bwd_scalars: s_t = bnd + sum_{t' >= t} r_t' per (b, h); ddt, dA/dD parts
// The running sums are kept in fp64: s_t sums thousands of terms of both signs
// to a small value, and dA sums dt_t s_t over the sequence again.
template <int L>
__global__ __launch_bounds__(256) void bwd_scalars_kernel(
    const float *__restrict__ tok, const float *__restrict__ DTws, const float *__restrict__ A,
    const double *__restrict__ bnd, float *__restrict__ ddt, double *__restrict__ part,
    int64_t T, int32_t H, int32_t nc, int64_t ntok, int64_t nbh) {
    // tiles of 2048 tokens from the last to the first; a thread takes 8
    // consecutive tokens of a tile (two 16-byte loads per plane, coalesced);
    // the tile's 256 segment sums are suffix-scanned within each wavefront by
    // lane shuffles and across the four wavefronts through LDS, and the
    // running carry holds the boundary term plus everything after the tile.
    // Each tile's planes are loaded while the previous tile is scanned.
    constexpr int TPT = 8, TT = 256 * TPT;
    __shared__ double wsum[2][4];
    __shared__ double red[2][4];
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H;
    const int32_t h = (int32_t)(bh % H);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t Tp = (int64_t)nc * L;             // padded tokens: r, x.U, dy.x, dt are 0
    const float *xu = tok + bh * Tp, *r = tok + ntok + bh * Tp, *dyx = tok + 2 * ntok + bh * Tp,
                *DT = DTws + bh * Tp;
    const double Ah = (double)A[h];
    double carry = bnd[bh], da = 0.0, dd = 0.0;
    float4 nv[4][2];                                 // planes r, x.U, dt, dy.x of the next tile
    auto load_tile = [&](int64_t tl) {
        const int64_t t0 = tl * TT + TPT * tid;
        const bool ok = tl >= 0 && t0 < Tp;          // Tp is a multiple of 64
        const float *src[4] = {r, xu, DT, dyx};
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                nv[k][u] = ok ? *reinterpret_cast<const float4 *>(src[k] + t0 + 4 * u)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    const int64_t ntl = (Tp + TT - 1) / TT;
    load_tile(ntl - 1);
    for (int64_t tl = ntl - 1; tl >= 0; --tl) {
        const int64_t t0 = tl * TT + TPT * tid;
        double rr[TPT], xx[TPT], dtt[TPT], yy[TPT];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float4 a = nv[0][u], x4 = nv[1][u], d4 = nv[2][u], y4 = nv[3][u];
            rr[4 * u] = a.x; rr[4 * u + 1] = a.y; rr[4 * u + 2] = a.z; rr[4 * u + 3] = a.w;
            xx[4 * u] = x4.x; xx[4 * u + 1] = x4.y; xx[4 * u + 2] = x4.z; xx[4 * u + 3] = x4.w;
            dtt[4 * u] = d4.x; dtt[4 * u + 1] = d4.y; dtt[4 * u + 2] = d4.z; dtt[4 * u + 3] = d4.w;
            yy[4 * u] = y4.x; yy[4 * u + 1] = y4.y; yy[4 * u + 2] = y4.z; yy[4 * u + 3] = y4.w;
        }
        load_tile(tl - 1);
        double seg = 0.0;
#pragma unroll
        for (int i = 0; i < TPT; ++i) seg += rr[i];
        // inclusive suffix sum over the wavefront's lanes
        double v = seg;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const double o = __shfl_down(v, d, 64);
            v += lane + d < 64 ? o : 0.0;
        }
        const int buf = (int)(tl & 1);
        if (lane == 0) wsum[buf][wv] = v;           // the wavefront's total
        __syncthreads();
        double after = 0.0, total = 0.0;            // later wavefronts' totals; the tile's
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const double t = wsum[buf][k];
            total += t;
            after += k > wv ? t : 0.0;
        }
        // the sum over every token after this thread's segment, then its tokens last to first
        double sfx = carry + after + (v - seg);
#pragma unroll
        for (int i = TPT - 1; i >= 0; --i) {
            sfx += rr[i];
            if (t0 + i < T) ddt[(b * T + t0 + i) * H + h] = (float)(xx[i] + Ah * sfx);
            da += dtt[i] * sfx;
            dd += yy[i];
        }
        carry += total;
    }
    // block sums of the dA and dD parts: wavefront shuffles, then the four
    // wavefronts in order
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
        da += __shfl_down(da, d, 64);
        dd += __shfl_down(dd, d, 64);
    }
    if (lane == 0) {
        red[0][wv] = da;
        red[1][wv] = dd;
    }
    __syncthreads();
    if (tid == 0) {
        part[bh] = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
        part[nbh + bh] = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
    }
}

// dA[h], dD[h]: the per-(b, h) parts summed over b in order
__global__ void bwd_heads_kernel(const double *__restrict__ part, float *__restrict__ dA,
                                 float *__restrict__ dD, int64_t Bt, int32_t H) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    double a = 0.0, d = 0.0;
    for (int64_t b = 0; b < Bt; ++b) {
        a += part[b * H + h];
        d += part[Bt * H + b * H + h];
    }
    dA[h] = (float)a;
    dD[h] = (float)d;
}

template <int L, int N, typename Tio, typename Thp>
hipError_t launch_bwd_t(const Shape &s, const BwdArgs &a, hipStream_t st) {
    const int64_t units = s.Bt * s.H * s.nc;
    const int64_t T = s.T;
    const int32_t H = (int32_t)s.H, G = (int32_t)s.G, nc = (int32_t)s.nc;
    const Tio *x = (const Tio *)a.x, *B = (const Tio *)a.B, *C = (const Tio *)a.C;
    if (units > 0 && !a.ghat_ready) {
        if constexpr (sizeof(Tio) == 2)
            hipLaunchKernelGGL((bwd_dstate_mfma_kernel<L, N>), dim3((uint32_t)units), dim3(256), 0,
                               st, a.dy, C, a.G, a.S, T, H, G, nc);
        else
            hipLaunchKernelGGL((bwd_dstate_kernel<L, N, Tio>), dim3((uint32_t)units), dim3(256), 0,
                               st, a.dy, C, a.G, a.S, T, H, G, nc);
    }
    // with ghat already in S only the boundary dot <dfinal, final> remains
    double *bnd = a.part + 2 * s.Bt * s.H;
    if (!a.ghat_ready)
        hipLaunchKernelGGL((bwd_passing_kernel<L, N>), dim3((uint32_t)(s.Bt * s.H)), dim3(256), 0,
                           st, a.S, a.G, a.dfinal, a.fin, a.dinit, bnd, nc);
    else if (a.dfinal)
        hipLaunchKernelGGL((bwd_bnd_kernel<N>), dim3((uint32_t)(s.Bt * s.H)), dim3(256), 0, st,
                           a.dfinal, a.fin, bnd);
    else
        hipLaunchKernelGGL((fill_f64_kernel), dim3((uint32_t)((s.Bt * s.H + 255) / 256)), dim3(256),
                           0, st, bnd, (int64_t)(s.Bt * s.H));
    if (units > 0) {
        constexpr int NTRI = (L / 64) * (L / 64 + 1) / 2;
        const uint64_t ncb = (uint64_t)s.Bt * s.nc * s.G;
        if constexpr (sizeof(Tio) == 2)
            hipLaunchKernelGGL((bwd_cb_mfma_kernel<L, N>), dim3((uint32_t)(ncb * NTRI)), dim3(256),
                               0, st, B, C, a.CB3, a.CBT3, T, G, nc);
        else
            hipLaunchKernelGGL((bwd_cb_kernel<L, N, Tio>), dim3((uint32_t)(ncb * NTRI)), dim3(256),
                               0, st, B, C, a.CB, T, G, nc);
        if constexpr (sizeof(Tio) == 2)
            hipLaunchKernelGGL((bwd_dx_mfma_kernel<L, N>), dim3((uint32_t)units),
                               dim3(4 * L), 0, st, x, B, C, a.D, a.dy, a.G, a.DT, a.CB3,
                               a.CBT3, (int64_t)(ncb * L * L), a.S,
                               (const float *)a.hprev, a.dx, a.tok, T, H, G, nc,
                               (int64_t)units * L);
        else
            hipLaunchKernelGGL((bwd_dx_kernel<L, N, Tio, Thp>), dim3((uint32_t)(units * (L / 64))),
                               dim3(256), 0, st, x, B, C, a.D, a.dy, a.G, a.DT, a.CB, a.S,
                               (const Thp *)a.hprev, a.dx, a.tok, T, H, G, nc);
        if constexpr (sizeof(Tio) == 2) {
            constexpr int WPB = L >= 128 ? 8 : 4;
            const uint32_t nb = (uint32_t)(ncb * (L / (16 * WPB)));
            hipLaunchKernelGGL((bwd_dc_mfma_kernel<L, N, WPB>), dim3(nb), dim3(64 * WPB), 0, st, x,
                               B, a.dy, a.G, a.DT, (const float *)a.hprev, a.dC, a.MT, T, H, G,
                               nc);
            hipLaunchKernelGGL((bwd_db_mfma_kernel<L, N, WPB>), dim3(nb), dim3(64 * WPB), 0, st, x,
                               C, a.G, a.DT, a.S, a.MT, a.dB, T, H, G, nc);
        } else {
            hipLaunchKernelGGL((bwd_dbdc_kernel<L, N, Tio, Thp>),
                               dim3((uint32_t)(ncb * (L / 64) * 2)), dim3(256), 0, st, x, B, C,
                               a.dy, a.G, a.DT, a.S, (const Thp *)a.hprev, a.dB, a.dC, T, H, G, nc);
        }
    }
    hipLaunchKernelGGL((bwd_scalars_kernel<L>), dim3((uint32_t)(s.Bt * s.H)), dim3(256), 0, st,
                       a.tok, a.DT, a.A, a.part + 2 * s.Bt * s.H, a.ddt, a.part, T, H, nc,
                       (int64_t)units * L, (int64_t)(s.Bt * s.H));
    hipLaunchKernelGGL(bwd_heads_kernel, dim3((uint32_t)((s.H + 63) / 64)), dim3(64), 0, st, a.part,
                       a.dA, a.dD, (int64_t)s.Bt, H);
    return hipGetLastError();
}

template <int L, int N>
hipError_t launch_bwd_ln(const Shape &s, const BwdArgs &a, hipStream_t st) {
    if (s.bf16) return launch_bwd_t<L, N, uint16_t, float>(s, a, st);
    return launch_bwd_t<L, N, float, float>(s, a, st);
}

template <int L>
hipError_t launch_bwd_l(const Shape &s, const BwdArgs &a, hipStream_t st) {
    if (s.N == 64) return launch_bwd_ln<L, 64>(s, a, st);
    if (s.N == 128) return launch_bwd_ln<L, 128>(s, a, st);
    return hipErrorInvalidValue;
}

}  // namespace

size_t bwd_cb_bytes(const Shape &s) { return (size_t)s.Bt * s.nc * s.G * s.L * s.L * 4; }

hipError_t launch_chunked_bwd(const Shape &s, const BwdArgs &a, hipStream_t st) {
    if (s.Bt == 0) return hipSuccess;
    if (s.L == 64) return launch_bwd_l<64>(s, a, st);
    if (s.L == 128) return launch_bwd_l<128>(s, a, st);
    if (s.L == 256) return launch_bwd_l<256>(s, a, st);
    return hipErrorInvalidValue;
}

}  // namespace ssd
