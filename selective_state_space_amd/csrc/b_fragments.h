// The state stage's B (or the adjoint's C) in MFMA fragment order, one
// workgroup's share: used by state_fwd's own launch and by the launch that
// builds the fragments next to the chunk cumsum.
#pragma once

#include <stdint.h>

#include "ssd_device.h"

namespace ssd {

// B of one (b, chunk, group) laid out as the MFMA B operand of the state
// product: fragment (slab js, n-tile nt) is 64 lanes x 16 bytes, lane
// (m, q) holding B[32 js + r(q, e)][n] for e = 0..7 and
// n = 64 (nt / 4) + 4 m + nt % 4, with the slab row r(q, e) = 8 q + e (plain
// order), or with PERM r(q, e) = 16 [e >= 4] + 4 q + e % 4, the K order of
// the fused forward's x fragments; with F16 the values are converted to fp16
// (round to nearest even, exact for bf16 values of fp16's normal range;
// magnitudes above 65504 saturate there).  Tokens past T are zero.  One
// workgroup per (b, chunk, group, slab) stages the 32 x N slab in LDS with
// coalesced 16-byte row loads and writes the N/16 fragments with 16-byte
// stores.
template <int L, int N, bool PERM = false, bool F16 = false>
__device__ __forceinline__ void b_fragments_block(const uint16_t *__restrict__ B,
                                                  uint4 *__restrict__ BF, int64_t T, int32_t G,
                                                  int32_t nc, int64_t blk) {
    // blk = ((b * nc + c) * G + g) * NS + js
    constexpr int NS = L / 32, NT = N / 16, RW = N / 8;   // 16-byte pieces per row
    __shared__ uint16_t tile[32][N + 8];
    const int js = (int)(blk % NS);
    const int64_t bcg = blk / NS;
    const int32_t g = (int32_t)(bcg % G);
    const int64_t bc = bcg / G;
    const int32_t c = (int32_t)(bc % nc);
    const int64_t b = bc / nc;
    const int tid = threadIdx.x;
    for (int k = tid; k < 32 * RW; k += 256) {
        const int r = k / RW, pc = k % RW;
        const int64_t tok = (int64_t)c * L + 32 * js + r;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (tok < T) v = *reinterpret_cast<const uint4 *>(B + ((b * T + tok) * G + g) * N + 8 * pc);
        *reinterpret_cast<uint4 *>(&tile[r][8 * pc]) = v;
    }
    __syncthreads();
    for (int k = tid; k < NT * 64; k += 256) {
        const int nt = k / 64, l = k % 64, m = l & 15, q = l >> 4;
        const int n = 64 * (nt >> 2) + 4 * m + (nt & 3);
        uint4 v;
        uint32_t *vw = reinterpret_cast<uint32_t *>(&v);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int e0 = 2 * rr, e1 = 2 * rr + 1;
            const int r0 = PERM ? 16 * (e0 >> 2) + 4 * q + (e0 & 3) : 8 * q + e0;
            const int r1 = PERM ? 16 * (e1 >> 2) + 4 * q + (e1 & 3) : 8 * q + e1;
            if constexpr (F16) {
                const float f0 = fminf(fmaxf(bf16_to_f32(tile[r0][n]), -65504.f), 65504.f);
                const float f1 = fminf(fmaxf(bf16_to_f32(tile[r1][n]), -65504.f), 65504.f);
                const f16x2_t hv = {(_Float16)f0, (_Float16)f1};
                vw[rr] = __builtin_bit_cast(uint32_t, hv);
            } else {
                vw[rr] = (uint32_t)tile[r0][n] | ((uint32_t)tile[r1][n] << 16);
            }
        }
        BF[blk * (NT * 64) + k] = v;
    }
}

}  // namespace ssd
