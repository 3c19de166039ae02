// state_passing: the sequential scan over chunks,
//     h_prev[c] = h;   h <- exp2(G_last,c) h + S_c;   final = h,
// starting from the initial state (or zeros).
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Kernel 2": the state entering each chunk is stored
// before the chunk's update, the sequential dependence stays inside one
// program while independent (batch, head, state-tile) slices run in
// parallel, and the state after the last chunk is the final state (fed back
// as the next call's initial state).  The "mamba3" kernel card ("Method")
// issues the chunk loads several chunks ahead of the carry that consumes them.
//
// The update is elementwise over the P*N state of each (b, h), so a thread
// owns 4 consecutive elements (one 16-byte load of S per chunk) and walks
// the chunks; loads run PF chunks ahead in a register ring so that the HBM
// latency overlaps the dependent chain.  h_prev is written in the io dtype
// (bf16 feeds the chunk_scan MFMA directly); the running state and the final
// state stay fp32.  init_state may alias final_state: each thread reads its
// elements before the loop and writes them after it.

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

constexpr int kPF = 8;  // chunks in flight per thread

template <int L, bool BF16>
__global__ __launch_bounds__(256) void state_passing_kernel(
    const float *__restrict__ S, const float *__restrict__ Gws, const float *init,
    void *__restrict__ hprev, float *fin, int32_t nc, int32_t PN, int32_t blocks_per_bh) {
    const int64_t bh = blockIdx.x / blocks_per_bh;
    const int32_t e = ((blockIdx.x % blocks_per_bh) * 256 + threadIdx.x) * 4;  // element
    if (e >= PN) return;

    float4 h = make_float4(0.f, 0.f, 0.f, 0.f);
    if (init) h = *reinterpret_cast<const float4 *>(init + bh * PN + e);

    const float *Sb = S + bh * (int64_t)nc * PN + e;
    const float *Gl = Gws + bh * (int64_t)nc * L + (L - 1);

    float4 sbuf[kPF];
    float gbuf[kPF];
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
        if (k < nc) {
            sbuf[k] = load_nt(Sb + (int64_t)k * PN);
            gbuf[k] = Gl[(int64_t)k * L];
        }
    }
    for (int32_t c0 = 0; c0 < nc; c0 += kPF) {
#pragma unroll
        for (int k = 0; k < kPF; ++k) {
            const int32_t c = c0 + k;
            if (c < nc) {
                const float4 s = sbuf[k];
                const float dec = fast_exp2(gbuf[k]);
                if (c + kPF < nc) {
                    sbuf[k] = load_nt(Sb + (int64_t)(c + kPF) * PN);
                    gbuf[k] = Gl[(int64_t)(c + kPF) * L];
                }
                // plain stores: chunk_scan reads h_prev next, and what it
                // finds in the memory-side cache is not read from HBM again
                const int64_t off = (bh * (int64_t)nc + c) * PN + e;
                if constexpr (BF16) {
                    uint2 v;
                    v.x = pack_bf16x2(h.x, h.y);
                    v.y = pack_bf16x2(h.z, h.w);
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(hprev) + off) = v;
                } else {
                    *reinterpret_cast<float4 *>(static_cast<float *>(hprev) + off) = h;
                }
                h.x = dec * h.x + s.x;
                h.y = dec * h.y + s.y;
                h.z = dec * h.z + s.z;
                h.w = dec * h.w + s.w;
            }
        }
    }
    if (fin) *reinterpret_cast<float4 *>(fin + bh * PN + e) = h;
}

template <int L>
hipError_t launch_sp(const Shape &s, const float *S, const float *Gws, const float *init,
                     void *hprev, float *fin, hipStream_t st) {
    const int32_t PN = (int32_t)(s.P * s.N);
    const int32_t bpb = (PN / 4 + 255) / 256;
    const uint64_t nblk = (uint64_t)s.Bt * s.H * bpb;
    if (s.bf16)
        hipLaunchKernelGGL((state_passing_kernel<L, true>), dim3((uint32_t)nblk), dim3(256), 0, st,
                           S, Gws, init, hprev, fin, (int32_t)s.nc, PN, bpb);
    else
        hipLaunchKernelGGL((state_passing_kernel<L, false>), dim3((uint32_t)nblk), dim3(256), 0,
                           st, S, Gws, init, hprev, fin, (int32_t)s.nc, PN, bpb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_passing(const Shape &s, const float *S, const float *Gws,
                                const float *init, void *hprev, float *fin, hipStream_t st) {
    if (s.Bt == 0) return hipSuccess;
    if (s.nc == 0 && !fin) return hipSuccess;
    switch (s.L) {
    case 64: return launch_sp<64>(s, S, Gws, init, hprev, fin, st);
    case 128: return launch_sp<128>(s, S, Gws, init, hprev, fin, st);
    case 256: return launch_sp<256>(s, S, Gws, init, hprev, fin, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
