// The state stage's B (or the adjoint's C) in MFMA fragment order, one
// workgroup's share: used by state_fwd's own launch and by the launch that
// builds the fragments next to the chunk cumsum.
#pragma once

#include <stdint.h>

#include "ssd_device.h"

namespace ssd {

// B of one (b, chunk, group) laid out as the MFMA B operand of the state
// product: fragment (slab js, n-tile nt) is 64 lanes x 16 bytes, lane
// (m, q) holding B[32 js + 8 q + e][n] for e = 0..7 and
// n = 64 (nt / 4) + 4 m + nt % 4.  Tokens past T are zero.  One workgroup per
// (b, chunk, group, slab) stages the 32 x N slab in LDS with coalesced 16-byte
// row loads and writes the N/16 fragments with 16-byte stores.
template <int L, int N>
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
        for (int rr = 0; rr < 4; ++rr)
            vw[rr] = (uint32_t)tile[8 * q + 2 * rr][n] | ((uint32_t)tile[8 * q + 2 * rr + 1][n] << 16);
        BF[blk * (NT * 64) + k] = v;
    }
}

}  // namespace ssd
