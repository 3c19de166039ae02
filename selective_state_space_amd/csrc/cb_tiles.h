// C B^T of one (b, chunk, group): the causal 16 x 16 tiles that the fused
// forward's intra-chunk product drains.
#pragma once

#include <stdint.h>

#include "ssd_device.h"

namespace ssd {

// Tiles of row block I come in pairs, one pair per 32-token slab js <= I / 2:
// (I, 2 js) and (I, 2 js + 1).  Pair slots of a (b, chunk, group) are laid
// out by row block: row block I starts at slot cb_pair_base(I), and
// cb_pair_base(L / 16) slots hold all of them.
__host__ __device__ constexpr int cb_pair_base(int I) { return ((I + 1) / 2) * ((I + 2) / 2); }

// The tiles (I, J), J <= I, of the L x L matrix (C B^T)_ij = C_i . B_j, one
// workgroup of 4 wavefronts per (b, chunk, group, part): wavefront w of part
// handles the row-block pair (I0, I1) = (pr, L/16 - 1 - pr), pr = 4 part + w,
// so every wavefront forms L/16 + 1 tiles.  Each tile is stored transposed in
// MFMA accumulator order: lane (m, q) of pair slot (I, js) holds 16 bytes, the
// bf16 (round to nearest even) of C_i . B_j for i = 16 I + m and
// j = 16 (2 js + u) + 4 q + e, e = 0..3, tile u = 0 in the low 8 bytes and
// u = 1 in the high 8 (zero where 2 js + 1 > I).  Both operands have the
// contraction index n contiguous in memory, so each lane reads its 16-byte
// pieces of B and C rows straight from global memory (rows past T read as
// zero).  ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels
// in NVIDIA CUDA Tile", section "Kernel 3": C B^T per chunk, which the heads
// of a group share.)
template <int L, int N>
__device__ __forceinline__ void cb_tiles_block(const uint16_t *__restrict__ B,
                                               const uint16_t *__restrict__ C,
                                               uint4 *__restrict__ CBT, int64_t T, int32_t G,
                                               int32_t nc, int64_t blk) {
    constexpr int NB = L / 16, NK = N / 32, NPAIR = NB / 2;
    constexpr int NPART = (NPAIR + 3) / 4, NSLOT = cb_pair_base(NB);
    const int part = (int)(blk % NPART);
    const int64_t bcg = blk / NPART;                 // (b * nc + c) * G + g
    const int32_t g = (int32_t)(bcg % G);
    const int64_t bc = bcg / G;
    const int32_t c = (int32_t)(bc % nc);
    const int64_t b = bc / nc;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int m = lane & 15, q = lane >> 4;
    const int pr = 4 * part + w;
    if (pr >= NPAIR) return;                         // wavefront-uniform
    const int64_t t0 = (int64_t)c * L;
    const int64_t rs = (int64_t)G * N;               // elements between token rows
    const uint16_t *cb = C + ((b * T + t0) * G + g) * N + 8 * q;
    const uint16_t *bb = B + ((b * T + t0) * G + g) * N + 8 * q;
    auto row = [&](const uint16_t *base, int r, int kn) {
        return (t0 + r < T) ? *reinterpret_cast<const uint4 *>(base + r * rs + 32 * kn)
                            : make_uint4(0u, 0u, 0u, 0u);
    };
    uint4 *out = CBT + bcg * (int64_t)(NSLOT * 64) + lane;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int I = k ? NB - 1 - pr : pr;
        bf16x8 ci[NK];
#pragma unroll
        for (int kn = 0; kn < NK; ++kn) ci[kn] = as_bf16x8(row(cb, 16 * I + m, kn));
        for (int js = 0; 2 * js <= I; ++js) {
            uint32_t wv[2][2] = {{0u, 0u}, {0u, 0u}};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int J = 2 * js + u;
                if (J > I) break;
                f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kn = 0; kn < NK; ++kn)
                    t = mfma16x16x32(as_bf16x8(row(bb, 16 * J + m, kn)), ci[kn], t);
                wv[u][0] = pack_bf16x2(t[0], t[1]);
                wv[u][1] = pack_bf16x2(t[2], t[3]);
            }
            out[(cb_pair_base(I) + js) * 64] = make_uint4(wv[0][0], wv[0][1], wv[1][0], wv[1][1]);
        }
    }
}

}  // namespace ssd
