// state_fwd: chunk_state and state_passing in one sequential pass over the
// chunks of each (b, h),
//     h_prev[c] = h;   h <- exp2(G_last,c) h + sum_j x_j (dt_j exp2(G_last,c - G_j)) B_j^T;
//     final = h.
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Kernel 2": one program per independent (batch, head,
// state tile) slice walks the chunks in order, stores the state entering each
// chunk, scales it by exp2 of the chunk's last cumulative decay and adds the
// chunk's product X^T (dt exp2(G_last - G) B) with the running state as the
// accumulator of the matrix product; after the last chunk the state is the
// final state.  The per-chunk states S_c of the four-stage form (section
// "Mamba-2 architecture", the jump formula) are never written to HBM: that
// saves a write and a read of Bt*H*nc*P*N fp32.
//
// gfx950 mapping (bf16 io only).  One workgroup of 4 wavefronts per (b, h,
// p-slab): the block owns the state rows p = 4M + s0 + s, s < SPB (SPB = 4,
// 2 or 1, the head's 64 rows split over 4/SPB workgroups when Bt*H alone
// would not fill the chip), all N columns.  The state lives in the MFMA
// accumulators (v_mfma_f32_16x16x32_bf16, K = tokens) for the block's whole
// life.  Per chunk:
//   1. store h_prev[c] (bf16) from the accumulators and scale them by
//      exp2(G_last);
//   2. w_j = dt_j exp2(G_last - G_j), one token per thread, into LDS;
//   3. build the x*w operand fragments (x is read along its slow axis: lanes
//      load SPB-wide row pieces of 8 tokens and pair them up in registers),
//      carried as a bf16 head plus a bf16 remainder (x*w is not exact in
//      bf16; one rounding costs up to 2^-9 of every term, too much for a
//      2e-2 rms bound on the final state where |h| runs far above its rms),
//      in LDS in fragment order;
//   4. run the MFMAs over the chunk's 32-token slabs.
// Steps 3 and 4 are software-pipelined by half chunks: the fragments of the
// next half are built (VALU) while the current half is multiplied (MFMA),
// from two LDS buffers, so the two units overlap inside each wavefront.
// B fragments (exact bf16, shared by the heads of a group and so
// L2-resident) come straight from global memory into registers, four slabs
// ahead: b_fragments_kernel lays B
//      out in fragment order beforehand (once per (b, chunk, group), in the
//      workspace region the four-stage form uses for S), so each is one
//      16-byte load with no transpose.
// x and B are read with buffer loads whose range is the chunk's valid rows:
// a ragged last chunk reads zeros past T (its dt is 0 there as well).
// Every exponent G_last - G_j and G_last is <= 0.
//
// The backward runs the same kernel in two more modes.  kModeF32 stores h_prev
// in fp32.  kModeAdjoint is the reverse scan of the state adjoint (the
// "mamba3" kernel card, section "Backward"): chunks last to first,
//     ghat[c] = g;   g <- exp2(G_last,c) g + sum_k (dy_k exp2(G_k)) C_k^T;
//     dinit = g,
// with dy (fp32) in place of x -- its weighted values carried, like x*w, as a
// bf16 head and remainder (a third term left the full-size dA where it was) --
// C fragments in place of B, dfinal as the initial state, and ghat stored in
// fp32.  Every exponent is again <= 0.

#include "b_fragments.h"
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

template <int L, int N, int SPB>
struct FwdCfg {
    static constexpr int NS = L / 32;                       // 32-token K slabs per chunk
    static constexpr int HS = NS / 2;                       // slabs per half chunk
    static constexpr int SW = SPB < 2 ? SPB : 2;            // row sets s per wavefront
    static constexpr int TW = SPB * (N / 16) / (4 * SW);    // n-tiles per wavefront
};

// Two half-chunk buffers of x*w fragments (the half being multiplied and the
// half being built) and the per-token weights of two chunks.
template <int L, int SPB, int NTERM>
struct FwdSmem {
    uint4 AF[2][L / 64][NTERM][SPB][64];  // half, slab of the half, bf16 term, row set s, lane
    float w[2][L];                    // by chunk parity
};

struct FwdArgs {
    const void *x;     // x (bf16), or dy (fp32) for the adjoint
    const uint4 *BF;   // B in MFMA fragment order, from b_fragments_kernel
    const float *Gws, *DTws, *init;
    void *hprev;       // bf16, or fp32 when the kernel's HP32 is set
    float *fin;
    int64_t T;
    int32_t H, G, nc, hpg;
};

// K consecutive bf16 (K = 4, 2, 1) as one or two 32-bit words, by a buffer
// load at byte offset off (0 past the resource's range).  AUX is the cache
// policy: kStream (nt) for data read once (x), 0 for data shared across
// workgroups through L2 (B).
constexpr int kStream = 2;
template <int K, int AUX = 0>
__device__ __forceinline__ uint2 load_bf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (K == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
        return make_uint2(v[0], v[1]);
    } else if constexpr (K == 2) {
        return make_uint2(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX), 0u);
    } else {
        return make_uint2((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX), 0u);
    }
}
// the word of element j of piece v
__device__ __forceinline__ uint32_t word_of(uint2 v, int j) { return (j < 2) ? v.x : v.y; }

// the three modes of state_fwd_kernel: the forward with bf16 or fp32 h_prev,
// and the adjoint scan of the backward
constexpr int kModeBf16 = 0, kModeF32 = 1, kModeAdjoint = 2;

// a lane's piece of SPB consecutive elements of one token row: SPB bf16 fit
// in two words; SPB fp32 take four words when SPB = 4
template <bool WIDE> struct XPiece { using type = uint2; };
template <> struct XPiece<true> { using type = uint4; };

// K consecutive fp32 (K = 4, 2, 1) by a buffer load, as in load_bf
template <int K, int AUX = 0>
__device__ __forceinline__ auto load_f32p(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (K == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
        return make_uint4(v[0], v[1], v[2], v[3]);
    } else if constexpr (K == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
        return make_uint2(v[0], v[1]);
    } else {
        return make_uint2(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX), 0u);
    }
}
// element j of a piece, as a float: bf16 pieces (two to a word) or fp32
__device__ __forceinline__ float elem_of(uint2 v, int j, bool f32) {
    if (f32) return __uint_as_float(j == 0 ? v.x : v.y);
    const uint32_t w = word_of(v, j);
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}
__device__ __forceinline__ float elem_of(uint4 v, int j, bool) {
    return __uint_as_float(j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w);
}

// K consecutive floats of a state row
template <int K>
__device__ __forceinline__ void load_f(const float *p, float *v) {
    if constexpr (K == 4) {
        const float4 t = *reinterpret_cast<const float4 *>(p);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else if constexpr (K == 2) {
        const float2 t = *reinterpret_cast<const float2 *>(p);
        v[0] = t.x; v[1] = t.y;
    } else {
        v[0] = *p;
    }
}
template <int K>
__device__ __forceinline__ void store_f(float *p, const float *v) {
    if constexpr (K == 4) *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else if constexpr (K == 2) *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
    else *p = v[0];
}
// Plain (not streaming) stores: chunk_scan reads h_prev right after this
// kernel, and lines left in the memory-side cache spare it that re-read from
// HBM (measured: the 2.7B forward takes 5% less time than with streaming stores).
template <int K>
__device__ __forceinline__ void store_bf(uint16_t *p, const float *v) {
    if constexpr (K == 4) *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    else if constexpr (K == 2) *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(v[0], v[1]);
    else *p = (uint16_t)f32_to_bf16_bits(v[0]);
}

// One workgroup per (b, chunk, group, slab): see b_fragments_block.
template <int L, int N>
__global__ __launch_bounds__(256) void b_fragments_kernel(const uint16_t *__restrict__ B,
                                                          uint4 *__restrict__ BF, int64_t T,
                                                          int32_t G, int32_t nc) {
    b_fragments_block<L, N>(B, BF, T, G, nc, blockIdx.x);
}

// One (b, h, row split) chain of the scan: lid is the workgroup's logical id.
template <int L, int N, int SPB, int MODE>
__device__ __forceinline__ void state_pass(const FwdArgs &a, uint32_t lid,
                                           FwdSmem<L, SPB, 2> &sm) {
    using Cfg = FwdCfg<L, N, SPB>;
    constexpr int P = 64, NS = Cfg::NS, HS = Cfg::HS, SW = Cfg::SW, TW = Cfg::TW;
    constexpr int PSPLIT = 4 / SPB;
    constexpr int NT = N / 16;
    constexpr bool ADJ = MODE == kModeAdjoint, HP32 = MODE != kModeBf16;
    constexpr int RD = ADJ ? 2 : 4;
    constexpr int R = NS < RD ? NS : RD;   // B ring depth (slabs in flight)
    constexpr int NTERM = 2;             // bf16 terms of the x*w (dy*w) operand
    constexpr int ES = ADJ ? 4 : 2;      // bytes per element of x (dy)
    using XP = typename XPiece<ADJ && SPB == 4>::type;
    // the chunk a step works on: in order, or last to first for the adjoint
    auto phys = [&](int32_t c) { return ADJ ? a.nc - 1 - c : c; };

    const int32_t ps = lid % PSPLIT;
    const uint32_t bh = lid / PSPLIT;
    const int32_t h = bh % a.H;
    const int64_t b = bh / a.H;
    const int32_t g = h / a.hpg;
    const int W = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tid = threadIdx.x, lane = tid & 63;
    const int m = lane & 15, q = lane >> 4;
    const int32_t XR = a.H * P;
    const bool builds = HS == 4 || W < HS;   // this wavefront builds a slab of each half

    // the block's rows: p = 4M + s0 + s (s < SPB); this wavefront's: s = sb + i
    // (i < SW); its columns: n = 64 (nt / 4) + 4m + nt % 4, nt = nt0 + j (j < TW)
    const int s0 = ps * SPB;
    const int sb = (SPB == 4) ? 2 * (W & 1) : 0;
    const int nt0 = TW * ((SPB == 4) ? (W >> 1) : W);
    const int ncol = 64 * (nt0 >> 2) + 4 * m + (nt0 & 3);   // first of TW columns
    auto prow = [&](int i, int e) { return 4 * (4 * q + e) + s0 + sb + i; };

    const int64_t bhi = (int64_t)b * a.H + h;
    f32x4 acc[SW][TW];
#pragma unroll
    for (int i = 0; i < SW; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v[TW];
            if (a.init) {
                load_f<TW>(a.init + (bhi * P + prow(i, e)) * N + ncol, v);
            } else {
#pragma unroll
                for (int j = 0; j < TW; ++j) v[j] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < TW; ++j) acc[i][j][e] = v[j];
        }
    if (a.nc == 0) {
        if (a.fin) {
#pragma unroll
            for (int i = 0; i < SW; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v[TW];
#pragma unroll
                    for (int j = 0; j < TW; ++j) v[j] = acc[i][j][e];
                    store_f<TW>(a.fin + (bhi * P + prow(i, e)) * N + ncol, v);
                }
        }
        return;
    }

    // Raw operands, loaded ahead of use and unconditionally (a load under a
    // branch, or one used right after issue, makes the compiler drain every
    // outstanding load with vmcnt(0) and serializes the chunks):
    //   xr[hf]  x pieces of the slab this wavefront builds in half hf, loaded
    //           two half-steps before that half is built;
    //   br      B fragments of this wavefront's columns, R slabs ahead (16
    //           bytes a lane each, from b_fragments_kernel);
    //   gv, dtv, glv  G and dt of token tid and the last G of the chunk after
    //           the one being multiplied.
    XP xr[2][8];
    bf16x8 br[R][TW];
    float gv = 0.f, dtv = 0.f, glv = 0.f;
    auto nvalid_of = [&](int32_t c) {
        const int64_t rem = a.T - (int64_t)c * L;
        return rem < L ? (int32_t)rem : L;
    };
    // Each chunk's x rows are read through a buffer resource that spans its
    // valid tokens only: rows past T (ragged last chunk) come back as 0.  The
    // row offset sits in the VGPR offset (the range check covers it); the
    // stride goes through an empty asm per call so that the offsets are
    // formed at each load rather than hoisted out of the chunk loop.
    // A chunk index past the last gives a resource of zero range: the loads
    // return zeros without touching memory (the pipeline's look-ahead past
    // the end costs no traffic and needs no branch).
    auto load_x = [&](int32_t c, int hf) {
        const bool real = c < a.nc;
        c = real ? phys(c) : a.nc - 1;
        const int32_t nv = real ? nvalid_of(c) : 0;
        int32_t rs = XR * ES;
        asm volatile("" : "+s"(rs));
        const auto rx = make_rsrc(static_cast<const char *>(a.x) +
                                      (((b * a.T + (int64_t)c * L) * a.H + h) * P + s0) * ES,
                                  (uint32_t)(nv * rs));
        const uint32_t lo = (uint32_t)(8 * q * rs + 4 * ES * m);
        const int js = HS * hf + W;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (ADJ)
                xr[hf][r] = load_f32p<SPB, kStream>(rx, lo + (uint32_t)((32 * js + r) * rs));
            else
                xr[hf][r] = load_bf<SPB, kStream>(rx, lo + (uint32_t)((32 * js + r) * rs));
        }
    };
    auto load_g = [&](int32_t c) {   // plain loads: the index is clamped
        const int64_t o = (bhi * a.nc + phys(min(c, a.nc - 1))) * L;
        gv = a.Gws[o + min(tid, L - 1)];
        dtv = a.DTws[o + min(tid, L - 1)];
        glv = a.Gws[o + L - 1];
    };
    auto load_b = [&](int32_t c, int js) {
        const bool real = c < a.nc;
        c = real ? phys(c) : a.nc - 1;
        const auto rb = make_rsrc(a.BF + (((b * a.nc + c) * a.G + g) * NS) * (NT * 64),
                                  real ? (uint32_t)(NS * NT * 64 * 16) : 0u);
#pragma unroll
        for (int j = 0; j < TW; ++j) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(
                rb, (uint32_t)(16 * lane), (uint32_t)(((js * NT + nt0 + j) * 64) * 16), 0);
            br[js % R][j] = __builtin_bit_cast(bf16x8, v);
        }
    };
    // x*w fragments of row set s of this wavefront's slab of half hf, with
    // weights w (8 tokens), into AF[hf]: a bf16 head plus a bf16 remainder
    // (the adjoint's dy*w: three bf16 terms)
    auto build_set = [&](int hf, int s, const float *w) {
        uint4 v[NTERM];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            float e0 = elem_of(xr[hf][2 * rr], s, ADJ) * w[2 * rr];
            float e1 = elem_of(xr[hf][2 * rr + 1], s, ADJ) * w[2 * rr + 1];
#pragma unroll
            for (int tm = 0; tm < NTERM; ++tm) {
                const uint32_t hw = pack_bf16x2(e0, e1);
                reinterpret_cast<uint32_t *>(&v[tm])[rr] = hw;
                e0 -= bf16_lo(hw);
                e1 -= bf16_hi(hw);
            }
        }
#pragma unroll
        for (int tm = 0; tm < NTERM; ++tm) sm.AF[hf][W][tm][s][lane] = v[tm];
    };
    auto read_w = [&](int hf, int wb, float *w) {
        const int jw = 32 * (HS * hf + W) + 8 * q;
        const float4 w0 = *reinterpret_cast<const float4 *>(&sm.w[wb][jw]);
        const float4 w1 = *reinterpret_cast<const float4 *>(&sm.w[wb][jw + 4]);
        w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
        w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
    };
    auto build = [&](int hf, int wb) {
        float w[8];
        read_w(hf, wb, w);
#pragma unroll
        for (int s = 0; s < SPB; ++s) build_set(hf, s, w);
    };
    // h += the products of half hf of chunk c, while (if bh >= 0) the x*w
    // fragments of half bh are built with the weights of buffer wb, one row
    // set per slab, interleaved with the MFMAs (VALU and matrix core work
    // from one wavefront overlap only when their instructions alternate).
    // The x*w fragments are read one slab ahead; B comes R slabs ahead
    // through the ring (slabs past the chunk's last come from chunk cn).
    auto mfma_half = [&](int hf, int32_t c, int32_t cn, int bh, int wb) {
        float w[8];
        if (bh >= 0 && builds) read_w(bh, wb, w);
        bf16x8 av[NTERM][SW];
#pragma unroll
        for (int hl = 0; hl < NTERM; ++hl)
#pragma unroll
            for (int i = 0; i < SW; ++i) av[hl][i] = as_bf16x8(sm.AF[hf][0][hl][sb + i][lane]);
#pragma unroll
        for (int k = 0; k < HS; ++k) {
            const int js = HS * hf + k;
            bf16x8 bfr[TW];
#pragma unroll
            for (int j = 0; j < TW; ++j) bfr[j] = br[js % R][j];
            if (js + R < NS) load_b(c, js + R);
            else load_b(cn, js + R - NS);
            bf16x8 an[NTERM][SW];
            if (k + 1 < HS) {
#pragma unroll
                for (int hl = 0; hl < NTERM; ++hl)
#pragma unroll
                    for (int i = 0; i < SW; ++i)
                        an[hl][i] = as_bf16x8(sm.AF[hf][k + 1][hl][sb + i][lane]);
            }
            if (bh >= 0 && builds) {
#pragma unroll
                for (int s = 0; s < SPB; ++s)
                    if (s % HS == k) build_set(bh, s, w);
            }
            // all head products, then all remainder products: no MFMA waits
            // on the one just issued
#pragma unroll
            for (int hl = 0; hl < NTERM; ++hl)
#pragma unroll
                for (int i = 0; i < SW; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j)
                        acc[i][j] = mfma16x16x32(av[hl][i], bfr[j], acc[i][j]);
            if (k + 1 < HS) {
#pragma unroll
                for (int hl = 0; hl < NTERM; ++hl)
#pragma unroll
                    for (int i = 0; i < SW; ++i) av[hl][i] = an[hl][i];
            }
            // schedule: the next slab's LDS reads and the B loads first, then
            // each MFMA followed by three VALU instructions of the fragment build
            __builtin_amdgcn_sched_group_barrier(0x100, NTERM * SW, 0);   // DS read
            __builtin_amdgcn_sched_group_barrier(0x020, TW, 0);       // VMEM read
#pragma unroll
            for (int u = 0; u < NTERM * SW * TW; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);    // VALU
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto store_hprev = [&](int32_t c) {
        const int64_t o = (bhi * a.nc + phys(c)) * (int64_t)(P * N) + ncol;
#pragma unroll
        for (int i = 0; i < SW; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v[TW];
#pragma unroll
                for (int j = 0; j < TW; ++j) v[j] = acc[i][j][e];
                if constexpr (HP32)
                    store_f<TW>(static_cast<float *>(a.hprev) + o + prow(i, e) * N, v);
                else
                    store_bf<TW>(static_cast<uint16_t *>(a.hprev) + o + prow(i, e) * N, v);
            }
    };

    // Prologue: weights of chunk 0, its first half built, x of its second
    // half and of chunk 1's first half in flight, G and dt of chunk 1.
    const int32_t c1 = 1;
    if (builds) {
        load_x(0, 0);
        load_x(0, 1);
    }
    load_g(0);
#pragma unroll
    for (int js = 0; js < R; ++js) load_b(0, js);
    float glc = glv;                 // last G of the chunk being multiplied
    if (tid < L) sm.w[0][tid] = ADJ ? fast_exp2(gv) : dtv * fast_exp2(glc - gv);
    load_g(c1);
    lds_barrier();
    if (builds) {
        build(0, 0);
        load_x(c1, 0);
    }

    // Steps of half a chunk.  In each, every wavefront builds the next half's
    // x*w fragments into one buffer while it multiplies the current half from
    // the other (the VALU work of one overlaps the MFMAs of the other), after
    // one barrier that publishes the half just built and frees the one just
    // multiplied.
    for (int32_t c = 0; c < a.nc; ++c) {
        const int32_t cn = c + 1, cnn = c + 2;   // may run past the end (zero-range loads)
        // ---- first half of chunk c (fragments in AF[0]) ----
        lds_barrier();
        store_hprev(c);              // the state entering chunk c
        const float dec = fast_exp2(glc);
#pragma unroll
        for (int i = 0; i < SW; ++i)
#pragma unroll
            for (int j = 0; j < TW; ++j) acc[i][j] *= dec;
        const float gln = glv;       // weights of chunk c + 1, then its G and dt in flight
        if (tid < L) sm.w[(c + 1) & 1][tid] = ADJ ? fast_exp2(gv) : dtv * fast_exp2(gln - gv);
        load_g(cnn);
        mfma_half(0, c, cn, 1, c & 1);   // and build the second half of chunk c
        if (builds) load_x(cn, 1);
        // ---- second half of chunk c (fragments in AF[1]) ----
        lds_barrier();
        mfma_half(1, c, cn, 0, (c + 1) & 1);   // and build the first half of chunk c + 1
        if (builds) load_x(cnn, 0);
        glc = gln;
    }
    if (a.fin) {
#pragma unroll
        for (int i = 0; i < SW; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v[TW];
#pragma unroll
                for (int j = 0; j < TW; ++j) v[j] = acc[i][j][e];
                store_f<TW>(a.fin + (bhi * P + prow(i, e)) * N + ncol, v);
            }
    }
}

template <int L, int N, int SPB, int MODE>
__global__ __launch_bounds__(256, 2) void state_fwd_kernel(FwdArgs a, uint32_t nblk) {
    __shared__ FwdSmem<L, SPB, 2> sm;
    state_pass<L, N, SPB, MODE>(a, xcd_remap(blockIdx.x, nblk), sm);
}

// The backward's two scans in one grid: workgroups [0, na) run the adjoint
// scan, [na, na + nf) recompute h_prev (fp32) and the final state.  The two
// are independent; sharing one grid lets the workgroups of each fill the
// slots the other leaves at its end, where two separate launches would each
// finish on a partly empty chip (Bt*H chains against two resident
// workgroups per CU).  The adjoint chains are the longer ones (fp32 dy), so
// they go first and the shorter recompute chains make up the last round.
template <int L, int N, int SPB>
__global__ __launch_bounds__(256, 2) void state_pair_kernel(FwdArgs af, FwdArgs aa, uint32_t nf,
                                                           uint32_t na) {
    __shared__ FwdSmem<L, SPB, 2> sm;
    const uint32_t bid = blockIdx.x;   // workgroup-uniform branch
    if (bid < na)
        state_pass<L, N, SPB, kModeAdjoint>(aa, xcd_remap(bid, na), sm);
    else
        state_pass<L, N, SPB, kModeF32>(af, xcd_remap(bid - na, nf), sm);
}

template <int L, int N, int SPB>
hipError_t launch_fwd(const Shape &s, const FwdArgs &a, int mode, hipStream_t st) {
    const uint64_t nblk = (uint64_t)s.Bt * s.H * (4 / SPB);
    if (mode == kModeAdjoint)
        hipLaunchKernelGGL((state_fwd_kernel<L, N, SPB, kModeAdjoint>), dim3((uint32_t)nblk),
                           dim3(256), 0, st, a, (uint32_t)nblk);
    else if (mode == kModeF32)
        hipLaunchKernelGGL((state_fwd_kernel<L, N, SPB, kModeF32>), dim3((uint32_t)nblk), dim3(256),
                           0, st, a, (uint32_t)nblk);
    else
        hipLaunchKernelGGL((state_fwd_kernel<L, N, SPB, kModeBf16>), dim3((uint32_t)nblk),
                           dim3(256), 0, st, a, (uint32_t)nblk);
    return hipGetLastError();
}

template <int L, int N>
hipError_t launch_fwd_n(const Shape &s, const FwdArgs &a, int spb, int mode, hipStream_t st) {
    switch (spb) {
    case 4: return launch_fwd<L, N, 4>(s, a, mode, st);
    case 2: return launch_fwd<L, N, 2>(s, a, mode, st);
    case 1: return launch_fwd<L, N, 1>(s, a, mode, st);
    default: return hipErrorInvalidValue;
    }
}

template <int L>
hipError_t launch_fwd_l(const Shape &s, const FwdArgs &a, int spb, int mode, hipStream_t st) {
    if (s.N == 64) return launch_fwd_n<L, 64>(s, a, spb, mode, st);
    if (s.N == 128) return launch_fwd_n<L, 128>(s, a, spb, mode, st);
    return hipErrorInvalidValue;
}

}  // namespace

int state_fwd_rows_per_block(const Shape &s) {
    // Row sets (of 16 state rows) per workgroup.  All four while Bt*H chains
    // alone give most of the 512 resident slots (two workgroups per CU);
    // fewer chains are split over 2 or 4 workgroups each, which also fit
    // three per CU, so that enough chains run at once.
    const int64_t bh = s.Bt * s.H;
    if (bh >= 384) return 4;
    if (bh >= 48) return 2;
    return 1;
}

bool state_fwd_preferred(const Shape &s) {
    // Measured on MI355X at the 370M, 2.7B and long-context shapes, the
    // one-pass form beats chunk_state + state_passing at each (it never
    // writes or reads the fp32 chunk states) once the row split keeps the
    // chains' sequential chunk steps overlapped.
    return state_fwd_supported(s);
}

bool state_fwd_supported(const Shape &s) {
    // per-chunk byte offsets of x rows are 32-bit
    const int64_t lim = (int64_t(1) << 31) - 1;
    return s.bf16 && s.P == 64 && s.L * s.H * s.P * 2 <= lim &&
           (uint64_t)s.Bt * s.nc * s.G * (s.L / 32) <= (uint64_t)lim;
}

size_t state_fwd_bfrag_bytes(const Shape &s) {
    return (size_t)s.Bt * s.nc * s.G * s.L * s.N * 2;
}

// the one-pass scan of either direction: x (or dy) and V = B (or C) in, the
// state before each chunk step (h_prev, or the adjoint ghat) and the last
// state (final, or dinit) out
// V (B or C, bf16) laid out in MFMA fragment order into vfrag
static hipError_t launch_vfrag(const Shape &s, const void *V, void *vfrag, hipStream_t st) {
    const uint64_t nfb = (uint64_t)s.Bt * s.nc * s.G * (s.L / 32);
    auto lb = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((uint32_t)nfb), dim3(256), 0, st, (const uint16_t *)V,
                           (uint4 *)vfrag, s.T, (int32_t)s.G, (int32_t)s.nc);
    };
    if (s.N == 64) {
        if (s.L == 64) lb(b_fragments_kernel<64, 64>);
        else if (s.L == 128) lb(b_fragments_kernel<128, 64>);
        else lb(b_fragments_kernel<256, 64>);
    } else {
        if (s.L == 64) lb(b_fragments_kernel<64, 128>);
        else if (s.L == 128) lb(b_fragments_kernel<128, 128>);
        else lb(b_fragments_kernel<256, 128>);
    }
    return hipGetLastError();
}

static FwdArgs pass_args(const Shape &s, const void *x, const void *vfrag, const float *Gws,
                         const float *DTws, const float *init, void *out, float *fin) {
    FwdArgs a;
    a.x = x;
    a.BF = (const uint4 *)vfrag;
    a.Gws = Gws;
    a.DTws = DTws;
    a.init = init;
    a.hprev = out;
    a.fin = fin;
    a.T = s.T;
    a.H = (int32_t)s.H;
    a.G = (int32_t)s.G;
    a.nc = (int32_t)s.nc;
    a.hpg = (int32_t)(s.H / s.G);
    return a;
}

// the one-pass scan of either direction: x (or dy) and V = B (or C) in, the
// state before each chunk step (h_prev, or the adjoint ghat) and the last
// state (final, or dinit) out
static hipError_t launch_pass(const Shape &s, const void *x, const void *V, const float *Gws,
                              const float *DTws, const float *init, void *out, float *fin,
                              void *vfrag, int spb, int mode, hipStream_t st,
                              bool vfrag_ready = false) {
    if (s.Bt == 0 || s.H == 0) return hipSuccess;
    if (s.nc == 0 && !fin) return hipSuccess;
    if (s.nc > 0 && !vfrag_ready) {
        const hipError_t e = launch_vfrag(s, V, vfrag, st);
        if (e != hipSuccess) return e;
    }
    const FwdArgs a = pass_args(s, x, vfrag, Gws, DTws, init, out, fin);
    switch (s.L) {
    case 64: return launch_fwd_l<64>(s, a, spb, mode, st);
    case 128: return launch_fwd_l<128>(s, a, spb, mode, st);
    case 256: return launch_fwd_l<256>(s, a, spb, mode, st);
    default: return hipErrorInvalidValue;
    }
}

template <int L, int N>
static hipError_t launch_pair_n(const Shape &s, const FwdArgs &af, const FwdArgs &aa, int spb,
                                hipStream_t st) {
    const uint32_t n = (uint32_t)(s.Bt * s.H * (4 / spb));
    auto lp = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(2 * n), dim3(256), 0, st, af, aa, n, n);
    };
    switch (spb) {
    case 4: lp(state_pair_kernel<L, N, 4>); break;
    case 2: lp(state_pair_kernel<L, N, 2>); break;
    case 1: lp(state_pair_kernel<L, N, 1>); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_state_fwd(const Shape &s, const void *x, const void *B, const float *Gws,
                            const float *DTws, const float *init, void *hprev, float *fin,
                            void *bfrag, int spb, bool hprev_f32, hipStream_t st,
                            bool bfrag_ready) {
    if (!state_fwd_supported(s)) return hipErrorInvalidValue;
    if (spb <= 0) spb = state_fwd_rows_per_block(s);
    return launch_pass(s, x, B, Gws, DTws, init, hprev, fin, bfrag, spb,
                       hprev_f32 ? kModeF32 : kModeBf16, st, bfrag_ready);
}

hipError_t launch_state_pair(const Shape &s, const void *x, const float *Gws, const float *DTws,
                             const float *init, float *hprev32, float *fin, const void *bfrag,
                             const float *dy, const void *C, const float *dfinal, float *ghat,
                             float *dinit, void *cfrag, int spb, hipStream_t st) {
    if (!state_adj_supported(s)) return hipErrorInvalidValue;
    if (spb <= 0) spb = state_fwd_rows_per_block(s);
    if (s.Bt == 0 || s.H == 0 || s.nc == 0) {   // nothing to overlap: the two scans alone
        hipError_t e = launch_pass(s, x, nullptr, Gws, DTws, init, hprev32, fin,
                                   const_cast<void *>(bfrag), spb, kModeF32, st, true);
        if (e != hipSuccess) return e;
        return launch_pass(s, dy, C, Gws, Gws, dfinal, ghat, dinit, cfrag, spb, kModeAdjoint, st);
    }
    hipError_t e = launch_vfrag(s, C, cfrag, st);
    if (e != hipSuccess) return e;
    const FwdArgs af = pass_args(s, x, bfrag, Gws, DTws, init, hprev32, fin);
    const FwdArgs aa = pass_args(s, dy, cfrag, Gws, Gws, dfinal, ghat, dinit);
    switch (s.L * 1000 + s.N) {
    case 64064: return launch_pair_n<64, 64>(s, af, aa, spb, st);
    case 64128: return launch_pair_n<64, 128>(s, af, aa, spb, st);
    case 128064: return launch_pair_n<128, 64>(s, af, aa, spb, st);
    case 128128: return launch_pair_n<128, 128>(s, af, aa, spb, st);
    case 256064: return launch_pair_n<256, 64>(s, af, aa, spb, st);
    case 256128: return launch_pair_n<256, 128>(s, af, aa, spb, st);
    default: return hipErrorInvalidValue;
    }
}

bool state_adj_supported(const Shape &s) {
    // as the forward, with fp32 dy rows
    const int64_t lim = (int64_t(1) << 31) - 1;
    return state_fwd_supported(s) && s.L * s.H * s.P * 4 <= lim;
}

int state_adj_rows_per_block(const Shape &s) {
    // the forward's rule: measured at the 2.7B shape, four row sets per
    // workgroup (one resident per CU: three bf16 terms take 1.5x the forward's
    // LDS) beat two (2.97 vs 3.03 ms for the whole backward) and one (3.26 ms)
    return state_fwd_rows_per_block(s);
}

hipError_t launch_state_adj(const Shape &s, const float *dy, const void *C, const float *Gws,
                            const float *dfinal, float *ghat, float *dinit, void *cfrag, int spb,
                            hipStream_t st) {
    if (!state_adj_supported(s)) return hipErrorInvalidValue;
    if (spb <= 0) spb = state_adj_rows_per_block(s);
    return launch_pass(s, dy, C, Gws, Gws, dfinal, ghat, dinit, cfrag, spb, kModeAdjoint, st);
}

}  // namespace ssd
