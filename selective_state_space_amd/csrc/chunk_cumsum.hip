// chunk_cumsum: G = log2(e) * chunk-local inclusive prefix sum of A_h dt_t.
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Kernel 1": the decay A*dt is summed cumulatively inside
// each chunk only (not over the whole sequence), once, for the two later
// stages; the sums are kept in log2 units so that later stages use exp2.  The
// same page's performance section stores dt and the cumulative decay head
// major, [batch, head, token], for contiguous per-head access: this kernel is
// where that transpose happens.
//
// Layout: reads dt [Bt, T, H] (heads contiguous); writes G and DT, both
// float32 [Bt, H, nc, L] (tokens contiguous).  Positions past T get dt = 0,
// so a ragged last chunk carries its last valid G to the end of the chunk.
//
// Optionally the step is preprocessed first, as the layer interface of
// "Optimizing Nemotron v3 Super in TensorRT-LLM" (sections 6.1, 6.3) does:
// dt <- dt + dt_bias_h, then dt <- log(1 + e^dt) where dt <= 20.  DT then
// holds the effective step, so the later stages need no change.
//
// One workgroup of 256 threads per (b, chunk, block of 16 heads).  dt rows of
// 16 heads (64 bytes) are read with 16-byte loads, transposed through LDS, and
// each wavefront then scans 4 heads: a lane sums L/64 tokens serially, a wave-wide
// log-depth scan (six DPP steps) combines the lane totals, and each lane
// adds its exclusive prefix back.

#include "b_fragments.h"
#include "cb_tiles.h"
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kHeadsPerBlock = 16;

// One workgroup's share: logical id lid -> (b, chunk, block of heads).
template <int L>
__device__ __forceinline__ void cumsum_block(
    const float *__restrict__ dt, const float *__restrict__ A, float *__restrict__ Gws,
    float *__restrict__ DTws, const float *__restrict__ dt_bias, int32_t softplus, int64_t T,
    int32_t H, int32_t nc, int32_t nhb, uint32_t lid) {
    constexpr int V = L / 64;  // tokens per lane
    __shared__ float tile[kHeadsPerBlock][L + 1];

    const int32_t hb = lid % nhb;
    const int32_t c = (lid / nhb) % nc;
    const int64_t b = lid / ((uint32_t)nhb * nc);
    const int32_t h0 = hb * kHeadsPerBlock;
    const int tid = threadIdx.x;

    // coalesced load of dt[b, c*L + t, h0 .. h0+KH-1]: KH/4 threads cover one
    // token row with 16-byte loads (when rows are 16-byte aligned)
    {
        constexpr int TPR = kHeadsPerBlock / 4, RPP = 256 / TPR;   // threads per row, rows per pass
        const int c4 = (tid % TPR) * 4;
        const bool vec = (H & 3) == 0;
#pragma unroll
        for (int k = 0; k < L / RPP; ++k) {
            const int t = tid / TPR + RPP * k;
            const int64_t tg = (int64_t)c * L + t;
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (tg < T) {
                const float *row = dt + (b * T + tg) * H + h0 + c4;
                if (vec && h0 + c4 + 3 < H) {
                    const float4 f = *reinterpret_cast<const float4 *>(row);
                    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (h0 + c4 + e < H) v[e] = row[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) tile[c4 + e][t] = v[e];
        }
    }
    __syncthreads();

    const int lane = tid & 63;
    const int wave = tid >> 6;
#pragma unroll
    for (int k = 0; k < kHeadsPerBlock / 4; ++k) {
        const int hh = wave + 4 * k;
        const int h = h0 + hh;
        if (h >= H) break;  // wave-uniform
        const float a2 = A[h] * kLog2e;
        const float bias = dt_bias ? dt_bias[h] : 0.f;
        float d[V], g[V];
        float run = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            d[v] = tile[hh][lane * V + v];
            if (dt_bias || softplus) {   // kernel-uniform
                const bool real = (int64_t)c * L + lane * V + v < T;   // padding stays 0
                float e = d[v] + bias;
                if (softplus && e <= 20.f) e = log1pf(expf(e));
                d[v] = real ? e : 0.f;
            }
            run += a2 * d[v];
            g[v] = run;
        }
        // inclusive scan of the lane totals across the wavefront
        const float incl = wave_inclusive_sum(run);
        const float excl = incl - run;
        const int64_t base = (((int64_t)b * H + h) * nc + c) * L + lane * V;
        if constexpr (V == 4) {
            *reinterpret_cast<float4 *>(Gws + base) =
                make_float4(g[0] + excl, g[1] + excl, g[2] + excl, g[3] + excl);
            *reinterpret_cast<float4 *>(DTws + base) = make_float4(d[0], d[1], d[2], d[3]);
        } else if constexpr (V == 2) {
            *reinterpret_cast<float2 *>(Gws + base) = make_float2(g[0] + excl, g[1] + excl);
            *reinterpret_cast<float2 *>(DTws + base) = make_float2(d[0], d[1]);
        } else {
            Gws[base] = g[0] + excl;
            DTws[base] = d[0];
        }
    }
}

template <int L>
__global__ __launch_bounds__(256) void chunk_cumsum_kernel(
    const float *__restrict__ dt, const float *__restrict__ A, float *__restrict__ Gws,
    float *__restrict__ DTws, const float *__restrict__ dt_bias, int32_t softplus, int64_t T,
    int32_t H, int32_t nc, int32_t nhb, uint32_t nblk) {
    cumsum_block<L>(dt, A, Gws, DTws, dt_bias, softplus, T, H, nc, nhb,
                    xcd_remap(blockIdx.x, nblk));
}

// The cumsum and the state stage's B fragments in one launch: both are small
// and independent, so one grid holds both sets of workgroups at once (the
// first ncum do the cumsum) and the forward pays one kernel boundary less.
template <int L, int N>
__global__ __launch_bounds__(256) void cumsum_bfrag_kernel(
    const float *__restrict__ dt, const float *__restrict__ A, float *__restrict__ Gws,
    float *__restrict__ DTws, const float *__restrict__ dt_bias, int32_t softplus, int64_t T,
    int32_t H, int32_t nc, int32_t nhb, uint32_t ncum, const uint16_t *__restrict__ B,
    uint4 *__restrict__ BF, int32_t G) {
    if (blockIdx.x < ncum)   // workgroup-uniform
        cumsum_block<L>(dt, A, Gws, DTws, dt_bias, softplus, T, H, nc, nhb,
                        xcd_remap(blockIdx.x, ncum));
    else
        b_fragments_block<L, N>(B, BF, T, G, nc, (int64_t)(blockIdx.x - ncum));
}

template <int L>
hipError_t launch_cumsum_bfrag(const Shape &s, const float *dt, const float *A, float *Gws,
                               float *DTws, const float *dt_bias, int softplus, int32_t nhb,
                               uint32_t ncum, const void *B, void *bfrag, hipStream_t st) {
    const uint64_t nfb = (uint64_t)s.Bt * s.nc * s.G * (L / 32);
    const dim3 grid((uint32_t)(ncum + nfb)), block(256);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, dt, A, Gws, DTws, dt_bias,
                           (int32_t)softplus, s.T, (int32_t)s.H, (int32_t)s.nc, nhb, ncum,
                           (const uint16_t *)B, (uint4 *)bfrag, (int32_t)s.G);
    };
    if (s.N == 64) go(cumsum_bfrag_kernel<L, 64>);
    else if (s.N == 128) go(cumsum_bfrag_kernel<L, 128>);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// Everything the fused forward needs before its sequential pass, in one
// launch of independent workgroups: the cumsum (first ncum), B in the fused
// pass's fragment order and in fp16 (next nbf), and the C B^T tiles (the rest).
template <int L, int N>
__global__ __launch_bounds__(256) void fused_prep_kernel(
    const float *__restrict__ dt, const float *__restrict__ A, float *__restrict__ Gws,
    float *__restrict__ DTws, const float *__restrict__ dt_bias, int32_t softplus, int64_t T,
    int32_t H, int32_t nc, int32_t nhb, uint32_t ncum, uint32_t nbf,
    const uint16_t *__restrict__ B, const uint16_t *__restrict__ C, uint4 *__restrict__ BF,
    uint4 *__restrict__ CBT, int32_t G) {
    if (blockIdx.x < ncum)   // workgroup-uniform
        cumsum_block<L>(dt, A, Gws, DTws, dt_bias, softplus, T, H, nc, nhb,
                        xcd_remap(blockIdx.x, ncum));
    else if (blockIdx.x < ncum + nbf)
        b_fragments_block<L, N, true, true>(B, BF, T, G, nc, (int64_t)(blockIdx.x - ncum));
    else
        cb_tiles_block<L, N>(B, C, CBT, T, G, nc, (int64_t)(blockIdx.x - ncum - nbf));
}

template <int L>
hipError_t launch_fused_prep_l(const Shape &s, const float *dt, const float *A, float *Gws,
                               float *DTws, const float *dt_bias, int softplus, const void *B,
                               const void *C, void *bfrag, void *cbt, hipStream_t st) {
    const int32_t nhb = (int32_t)((s.H + kHeadsPerBlock - 1) / kHeadsPerBlock);
    const uint64_t ncum = (uint64_t)s.Bt * s.nc * nhb;
    const uint64_t bcg = (uint64_t)s.Bt * s.nc * s.G;
    const uint64_t nbf = bcg * (L / 32);
    const uint64_t ncb = bcg * ((L / 32 + 3) / 4);
    const uint64_t total = ncum + nbf + ncb;
    if (total > 0x7fffffffull) return hipErrorInvalidValue;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((uint32_t)total), dim3(256), 0, st, dt, A, Gws, DTws,
                           dt_bias, (int32_t)softplus, s.T, (int32_t)s.H, (int32_t)s.nc, nhb,
                           (uint32_t)ncum, (uint32_t)nbf, (const uint16_t *)B,
                           (const uint16_t *)C, (uint4 *)bfrag, (uint4 *)cbt, (int32_t)s.G);
    };
    if (s.N == 64) go(fused_prep_kernel<L, 64>);
    else if (s.N == 128) go(fused_prep_kernel<L, 128>);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fused_prep(const Shape &s, const float *dt, const float *A, float *Gws,
                             float *DTws, const float *dt_bias, int softplus, const void *B,
                             const void *C, void *bfrag, void *cbt, hipStream_t st) {
    if (s.Bt == 0 || s.nc == 0) return hipSuccess;
    switch (s.L) {
    case 64: return launch_fused_prep_l<64>(s, dt, A, Gws, DTws, dt_bias, softplus, B, C, bfrag,
                                            cbt, st);
    case 128: return launch_fused_prep_l<128>(s, dt, A, Gws, DTws, dt_bias, softplus, B, C,
                                              bfrag, cbt, st);
    case 256: return launch_fused_prep_l<256>(s, dt, A, Gws, DTws, dt_bias, softplus, B, C,
                                              bfrag, cbt, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_cumsum(const Shape &s, const float *dt, const float *A, float *Gws,
                               float *DTws, const float *dt_bias, int softplus, hipStream_t st,
                               const void *B, void *bfrag) {
    if (s.Bt == 0 || s.nc == 0) return hipSuccess;
    const int32_t nhb = (int32_t)((s.H + kHeadsPerBlock - 1) / kHeadsPerBlock);
    const uint64_t nblk = (uint64_t)s.Bt * s.nc * nhb;
    if (bfrag) {
        switch (s.L) {
        case 64: return launch_cumsum_bfrag<64>(s, dt, A, Gws, DTws, dt_bias, softplus, nhb,
                                                (uint32_t)nblk, B, bfrag, st);
        case 128: return launch_cumsum_bfrag<128>(s, dt, A, Gws, DTws, dt_bias, softplus, nhb,
                                                  (uint32_t)nblk, B, bfrag, st);
        case 256: return launch_cumsum_bfrag<256>(s, dt, A, Gws, DTws, dt_bias, softplus, nhb,
                                                  (uint32_t)nblk, B, bfrag, st);
        default: return hipErrorInvalidValue;
        }
    }
    const dim3 grid((uint32_t)nblk), block(256);
    switch (s.L) {
    case 64:
        hipLaunchKernelGGL(chunk_cumsum_kernel<64>, grid, block, 0, st, dt, A, Gws, DTws, dt_bias,
                           (int32_t)softplus, s.T, (int32_t)s.H, (int32_t)s.nc, nhb,
                           (uint32_t)nblk);
        break;
    case 128:
        hipLaunchKernelGGL(chunk_cumsum_kernel<128>, grid, block, 0, st, dt, A, Gws, DTws, dt_bias,
                           (int32_t)softplus, s.T, (int32_t)s.H, (int32_t)s.nc, nhb,
                           (uint32_t)nblk);
        break;
    case 256:
        hipLaunchKernelGGL(chunk_cumsum_kernel<256>, grid, block, 0, st, dt, A, Gws, DTws, dt_bias,
                           (int32_t)softplus, s.T, (int32_t)s.H, (int32_t)s.nc, nhb,
                           (uint32_t)nblk);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssd
