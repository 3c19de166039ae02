// Device-side helpers shared by the SSD kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr float kLog2e = 1.4426950408889634f;

// MFMA operand / accumulator registers.
typedef short bf16x8 __attribute__((ext_vector_type(8)));  // 8 bf16, 4 VGPRs
typedef float f32x4 __attribute__((ext_vector_type(4)));   // 16x16 accumulator slice

// bf16 <-> float.  bf16 is carried as its 16-bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return pack_bf16x2(f, 0.f) & 0xffffu;
}

// fp16 operands (the fused forward's chunk-state product)
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));   // 8 fp16, 4 VGPRs
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const f16x2_t v = {(_Float16)lo, (_Float16)hi};   // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

// Streaming 16/8-byte accesses (nontemporal hint) for data that one call
// touches exactly once: the state slabs S, h_prev, y and the decode state.
// They keep such streams from displacing reused lines in L2 / the MALL.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 load_nt(const float *p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 load_nt(const uint16_t *p) {   // 4 bf16
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    return make_uint2(v[0], v[1]);
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt8(const uint16_t *p) {  // 8 bf16
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_nt(float *p, float4 v) {
    const f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ void store_nt(float *p, float2 v) {
    const f32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x2 *>(p));
}
__device__ __forceinline__ void store_nt(uint16_t *p, uint2 v) {
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2 *>(p));
}
__device__ __forceinline__ void store_nt(uint16_t *p, uint4 v) {   // 8 16-bit elements
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

// Output stores: y in float32, or in bf16 (round to nearest even) when the
// caller asked for y in the io dtype.  ybf is uniform over the launch.
__device__ __forceinline__ void store_y1(void *y, int64_t i, float v, bool ybf) {
    if (ybf)
        static_cast<uint16_t *>(y)[i] = (uint16_t)f32_to_bf16_bits(v);
    else
        static_cast<float *>(y)[i] = v;
}
// four consecutive outputs from element i (16- or 8-byte aligned), streaming
__device__ __forceinline__ void store_y4(void *y, int64_t i, float4 v, bool ybf) {
    if (ybf)
        store_nt(static_cast<uint16_t *>(y) + i, make_uint2(pack_bf16x2(v.x, v.y),
                                                            pack_bf16x2(v.z, v.w)));
    else
        store_nt(static_cast<float *>(y) + i, v);
}

// Workgroup barrier for LDS hand-offs only: the wavefront's LDS operations
// have completed (lgkmcnt 0), then s_barrier.  __syncthreads() also waits for
// every outstanding global load and store of the wavefront (vmcnt 0: its
// workgroup-scope fence), which would end every prefetch in flight at each
// barrier; kernels that exchange only LDS data between wavefronts use this.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 4 (or 1) io-dtype values as fp32: float, or bf16 carried as uint16_t.
template <typename Tio>
__device__ __forceinline__ float4 load4(const Tio *p);
template <>
__device__ __forceinline__ float4 load4<float>(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}
template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t *p) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    return make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
}
__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t *p) { return bf16_to_f32(*p); }

// silu(z) = z / (1 + e^-z) on the transcendental unit: e^-z as 2^(-z log2 e),
// then v_rcp_f32.  Both limits come out right: z -> -inf gives 1/inf = 0 and
// z -> +inf gives z * 1.
__device__ __forceinline__ float fast_silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.f + fast_exp2(-1.4426950408889634f * z));
}

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Map the
// hardware id to a logical id so that consecutive logical ids share an XCD
// (and its L2): logical [x*per, (x+1)*per) runs on XCD x.  Ids past the last
// multiple of 8 map to themselves.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nblk) {
    const uint32_t full = nblk & ~7u;
    if (bid >= full) return bid;
    const uint32_t per = full >> 3;
    return (bid & 7u) * per + (bid >> 3);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Transpose helpers for building MFMA operands from row-major tiles.
// Given two 32-bit words each holding a bf16 pair (lo = element 0, hi =
// element 1) from two consecutive rows r0, r1, produce the word holding
// element 0 of both rows, or element 1 of both rows.
// One v_perm_b32 each (byte selectors: 0-3 pick bytes of r0, 4-7 of r1).
__device__ __forceinline__ uint32_t pair_lo(uint32_t r0, uint32_t r1) {
    return __builtin_amdgcn_perm(r1, r0, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t r0, uint32_t r1) {
    return __builtin_amdgcn_perm(r1, r0, 0x07060302u);
}

// Raw buffer resource over `bytes` bytes from `base` (gfx9 dword3).  Loads at
// a VGPR offset at or past `bytes` return 0 without touching memory (the
// buffer range check), which is how ragged chunks read their missing rows.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Sum over each group of LPR = 8, 16 or 32 consecutive lanes by DPP moves
// (VALU operand modifiers, no LDS crossbar round trip): butterflies inside
// quads, then the half-row mirror leaves every lane of an 8-lane group with
// its sum, the row mirror every lane of a 16-lane row; for 32-lane groups,
// row_bcast:15 adds row 0's (row 2's) sum into row 1 (row 3).  The group's sum
// is valid in its last lane, LPR - 1 (for LPR = 8 and 16, in every lane).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "8-, 16- or 32-lane groups");
    v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);   // row_half_mirror
    if constexpr (LPR >= 16) v += dpp_mov<0x140>(v);   // row_mirror
    if constexpr (LPR == 32) v += dpp_mov<0x142, 0xa>(v);   // row_bcast:15 into rows 1, 3
    return v;
}
// Inclusive prefix sum over the 64 lanes of a wavefront by DPP moves: shifts
// by 1, 2, 4 and 8 lanes inside each 16-lane row (lanes shifted in read 0),
// then row_bcast:15 carries each even row's total into the row after it and
// row_bcast:31 the first half's total into the second half.
__device__ __forceinline__ float wave_inclusive_sum(float v) {
    v += dpp_mov<0x111>(v);         // row_shr:1
    v += dpp_mov<0x112>(v);         // row_shr:2
    v += dpp_mov<0x114>(v);         // row_shr:4
    v += dpp_mov<0x118>(v);         // row_shr:8
    v += dpp_mov<0x142, 0xa>(v);    // row_bcast:15 into rows 1, 3
    v += dpp_mov<0x143, 0xc>(v);    // row_bcast:31 into rows 2, 3
    return v;
}
// The maximum over each group of LPR = 8, 16 or 32 lanes, in every lane of it:
// the same DPP steps within 8- or 16-lane groups, then one swap of
// neighbouring rows.
template <int LPR>
__device__ __forceinline__ float group_max(float v) {
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "8-, 16- or 32-lane groups");
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    if constexpr (LPR >= 16) v = fmaxf(v, dpp_mov<0x140>(v));
    if constexpr (LPR == 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
    return v;
}

}  // namespace ssd
