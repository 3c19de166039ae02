// fused_fwd: the chunked forward after the cumsum as ONE sequential pass per
// (b, h) chain.  For each chunk c in order, with h the state entering it:
//     y_c  = exp2(G) C h^T + (exp2(G_i - G_j) (C B^T)_ij dt_j [j <= i]) X + D X
//     h   <- exp2(G_last) h + X^T diag(dt exp2(G_last - G)) B
// and final = h after the last chunk.
//
// "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Mamba-2 architecture" (the chunked output and the jump
// of the state over a chunk), section "Kernel 2" (one program walks the chunks
// of an independent slice in order, the state being the accumulator of the
// per-chunk product) and section "Kernel 3" (the chunk output from the state
// entering the chunk, with C B^T decayed and causally masked on chip).  Here
// the two are one pass: the state never leaves the chip between chunks, so
// neither the per-chunk states nor h_prev travel through HBM, and x is read
// once.  The "mamba3" kernel card ("Method") folds the decay and the causal
// weight into the drain of C B^T.
//
// gfx950 mapping (bf16 io): one workgroup of NW = L/32 wavefronts per (b, h).
// Wavefront W owns
//   - the output row blocks I0 = W and I1 = L/16 - 1 - W (16 tokens each; the
//     pair holds L/16 + 1 causal C B^T tiles for every W), all 64 columns p;
//   - SPW x NTW tiles (16 x 16) of the P x N state, held in MFMA accumulators
//     for the workgroup's whole life;
//   - slab W (32 tokens) of each chunk's x, which it loads and stages.
// Per chunk, two phases separated by barriers:
//   A. (reads the chunk's LDS buffers) scale the state by exp2(G_last); the
//      inter product C h^T from the h fragments (rows then scaled by
//      exp2(G_i)); then per 32-token slab the state product (x w) B -- w =
//      dt exp2(G_last - G), x w rounded once to fp16 and B in fp16
//      (v_mfma_f32_16x16x32_f16: fp16's 11-bit significand is what lets one
//      term do here what the one-pass state stage needs a bf16 head and
//      remainder for) -- and the intra product: each cached C B^T
//      tile drained in registers (times exp2(G_i - G_j) dt_j, factored through
//      the block's last token below the diagonal, exact with a causal select
//      on it) straight into the A operand; finally y = acc + D x (and the
//      optional gate), stored fp32 or bf16.
//   B. stage the next chunk into LDS: x fragments and (x w) fragments of slab
//      W, its G, dt and column factors V, and the state h (bf16) as the B
//      operand of the next inter product; then issue the next chunk's C
//      fragments, C B^T tiles and first B fragments.
// Operands: C B^T (per (b, chunk, group), bf16, 16x16 tiles in accumulator
// order) and B (in MFMA fragment order, K in the slot order of the x
// fragments) are laid out beforehand by the prepass, once per group, and come
// from L2 / the memory-side cache (a group's heads run on one XCD); C rows
// come straight from global memory (the contraction index n is contiguous).
// x is loaded one chunk ahead; every load is unconditional (a chunk index past
// the last reads through a zero-range buffer resource or is clamped), so the
// compiler never drains the queue early.  Ragged last chunk: x and C rows past
// T read as zero (buffer range check), dt is 0 there, y rows past T are not
// stored.  Every exponent used is <= 0.

#include "cb_tiles.h"
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

template <int L, int N>
struct FusedCfg {
    static constexpr int P = 64;
    static constexpr int NW = L / 32;         // wavefronts (one row-block pair and one slab each)
    static constexpr int NB = L / 16;         // 16-token row blocks
    static constexpr int NS = L / 32;         // 32-token K slabs
    static constexpr int NK = N / 32;         // K steps of the inter product
    static constexpr int NT = N / 16;         // 16-column n-tiles of the state
    static constexpr int TPW = 4 * NT / NW;   // state tiles per wavefront
    static constexpr int SPW = TPW / 2 < 4 ? TPW / 2 : 4;   // row sets s per wavefront
    static constexpr int NTW = TPW / SPW;     // n-tiles per wavefront (2 or 4, adjacent columns)
    static constexpr int SG = 4 / SPW;        // wavefronts sharing an n-tile group
    static constexpr int NPW = NB / 2 + 1;    // C B^T tile pairs per wavefront
    static constexpr int NSLOT = cb_pair_base(NB);   // tile pairs per (b, chunk, group)
    static constexpr int R = NS < 4 ? NS : 4; // B-fragment ring (slabs in flight)
    static_assert(SPW * NTW == TPW && SG * (NT / NTW) == NW, "state tile split");
    static_assert(NTW == 2 || NTW == 4, "adjacent column pairs or quads");
};

template <int L, int N>
struct FusedSmem {
    using Cfg = FusedCfg<L, N>;
    uint4 XF[Cfg::NS][4][64];   // x (bf16): slab js, row set s; lane (m, q) holds x[slot(q, e)][4m + s]
    uint4 AF[Cfg::NS][4][64];   // x w (fp16), same layout
    uint4 HF[Cfg::NK][4][64];   // h (bf16): lane (m, q) holds h[4m + s][32 kn + 8q + e]
    float G[L], V[L], DT[L];
};
// Each wavefront's C B^T tile pairs, written only by direct global-to-LDS
// loads: a separate LDS object, so that the compiler's wait for those loads
// is not attached to reads and writes of the other buffers.
template <int L>
struct FusedCbSmem {
    uint4 CB[L / 32][L / 32 + 1][64];
};

struct FusedArgs {
    const uint16_t *x, *C, *z;
    const uint4 *BF;          // B fragments (fp16) [b][chunk][group][slab][n-tile][64]
    const uint4 *CBT;         // C B^T tile pairs [b][chunk][group][pair slot][64]
    const float *D, *Gws, *DTws, *init;
    float *fin;
    void *y;                  // float32, or bf16 in the YBF instantiations
    int64_t T;
    int32_t H, G, nc, hpg;
};

constexpr int kStream = 2;   // buffer-load cache policy: nontemporal (data read once)

__device__ __forceinline__ f16x8 as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }


template <int L, int N, bool GATE, bool YBF, int W>
__device__ __forceinline__ void fused_body(FusedSmem<L, N> &sm, FusedCbSmem<L> &cbs,
                                           const FusedArgs &a, int64_t b, int32_t h) {
    using Cfg = FusedCfg<L, N>;
    constexpr int P = 64, NB = Cfg::NB, NS = Cfg::NS, NK = Cfg::NK, NT = Cfg::NT;
    constexpr int SPW = Cfg::SPW, NTW = Cfg::NTW, SG = Cfg::SG, R = Cfg::R;
    constexpr int NSLOT = Cfg::NSLOT;
    constexpr int I0 = W, I1 = NB - 1 - W;        // this wavefront's row blocks (I0 < I1)
    constexpr int N0 = I0 / 2 + 1;                // tile pairs of I0 (then those of I1)
    constexpr int S0 = SPW * (W % SG), NT0 = NTW * (W / SG);
    // in-loop issue point (slab index) of the next x: after the last B load
    // of this chunk
    constexpr int XLOAD_AT = NS > R ? NS - R - 1 : 0;
    // the lane index, refreshed through an opaque copy in each chunk (below):
    // the per-lane offsets derived from it are recomputed there instead of
    // being hoisted out of the chunk loop, where they would all stay live
    int lane = threadIdx.x & 63, m = lane & 15, q = lane >> 4;
    const int32_t g = h / a.hpg;
    const int64_t bh = b * a.H + h;
    const int32_t XR = a.H * P;                   // elements between token rows of x (and y, z)
    const int32_t CR = a.G * N;                   // of C
    const float Dh = a.D[h];
    // the first of this lane's NTW adjacent state columns; its state rows are
    // p = 4 (4q + e) + S0 + i
    int ncol = 64 * (NT0 >> 2) + 4 * m + (NT0 & 3);
    auto nvalid_of = [&](int32_t c) -> int32_t {
        const int64_t rem = a.T - (int64_t)c * L;
        return rem < L ? (int32_t)rem : L;
    };

    // ---- the state, from init_state (or zeros) ----
    f32x4 accs[SPW][NTW];
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p = 4 * (4 * q + e) + S0 + i;
            float v[NTW];
            if (a.init) {
                const float *src = a.init + (bh * P + p) * N + ncol;
                if constexpr (NTW == 2) {
                    const float2 t = *reinterpret_cast<const float2 *>(src);
                    v[0] = t.x; v[1] = t.y;
                } else {
                    const float4 t = *reinterpret_cast<const float4 *>(src);
                    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < NTW; ++j) v[j] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < NTW; ++j) accs[i][j][e] = v[j];
        }
    auto store_final = [&]() {
#pragma unroll
        for (int i = 0; i < SPW; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float *dst = a.fin + (bh * P + 4 * (4 * q + e) + S0 + i) * N + ncol;
                if constexpr (NTW == 2)
                    *reinterpret_cast<float2 *>(dst) = make_float2(accs[i][0][e], accs[i][1][e]);
                else
                    *reinterpret_cast<float4 *>(dst) = make_float4(
                        accs[i][0][e], accs[i][1][e], accs[i][2][e], accs[i][3][e]);
            }
    };
    if (a.nc == 0) {
        if (a.fin) store_final();
        return;
    }

    // ---- loads ----
    // x of slab W of a chunk (8 token rows, 4 columns 4m..4m+3 per lane), and
    // G and dt of this lane's 8 slots: slot e of lane q is token
    // 32 W + 16 [e >= 4] + 4 q + e % 4.  A chunk index past the last reads x
    // through a zero-range resource (zeros, no traffic) and G / dt of the
    // last chunk again.
    uint2 xr[8];
    float4 gq[2], dq[2];
    float glx;                                    // G at the last token of that chunk
    auto load_x = [&](int32_t c) {
        const bool real = c < a.nc;
        const int32_t cc = real ? c : a.nc - 1;
        const int32_t nv = real ? nvalid_of(cc) : 0;
        const uint32_t rs = (uint32_t)XR * 2u;
        const auto rx = make_rsrc(a.x + ((b * a.T + (int64_t)cc * L) * a.H + h) * P,
                                  (uint32_t)nv * rs);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const uint32_t tl = 32 * W + 16 * (rr >> 2) + 4 * q + (rr & 3);
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rx, tl * rs + 8u * m, 0, kStream);
            xr[rr] = make_uint2(v[0], v[1]);
        }
        const int64_t o = (bh * a.nc + cc) * L;
        gq[0] = *reinterpret_cast<const float4 *>(a.Gws + o + 32 * W + 4 * q);
        gq[1] = *reinterpret_cast<const float4 *>(a.Gws + o + 32 * W + 16 + 4 * q);
        dq[0] = *reinterpret_cast<const float4 *>(a.DTws + o + 32 * W + 4 * q);
        dq[1] = *reinterpret_cast<const float4 *>(a.DTws + o + 32 * W + 16 + 4 * q);
        glx = a.Gws[o + L - 1];
    };
    // B fragments of slab js of chunk c into the ring slot js % R, and the C
    // fragments of the two row blocks (c is clamped to the last chunk: loads
    // past the end only repeat it)
    uint4 cfr[2][NK];
    f16x8 bfr[R][NTW];
    auto load_b = [&](int32_t c, int js) {
        c = min(c, a.nc - 1);
        const uint4 *bp = a.BF + ((((b * a.nc + c) * a.G + g) * NS + js) * NT + NT0) * 64 + lane;
#pragma unroll
        for (int j = 0; j < NTW; ++j) bfr[js % R][j] = as_f16x8(bp[j * 64]);
    };
    auto load_c = [&](int32_t c) {
        c = min(c, a.nc - 1);
        const int32_t nv = nvalid_of(c);
        const auto rc = make_rsrc(a.C + ((b * a.T + (int64_t)c * L) * a.G + g) * N,
                                  (uint32_t)nv * (uint32_t)CR * 2u);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int I = k ? I1 : I0;
#pragma unroll
            for (int kn = 0; kn < NK; ++kn) {
                const uint32_t off = ((uint32_t)(16 * I + m) * (uint32_t)CR + 32 * kn + 8 * q) * 2u;
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
                cfr[k][kn] = make_uint4(v[0], v[1], v[2], v[3]);
            }
        }
    };
    // this wavefront's C B^T tile pairs of chunk c, straight into its own LDS
    // slots (global_load_lds, 16 bytes a lane): read only by this wavefront,
    // after an explicit wait for its vector-memory counter
    auto load_cb = [&](int32_t c) {
        c = min(c, a.nc - 1);
        const uint4 *src = a.CBT + ((b * a.nc + c) * a.G + g) * (int64_t)(NSLOT * 64) + lane;
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int I = k ? I1 : I0;
#pragma unroll
            for (int js = 0; 2 * js <= I; ++js)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(src + (cb_pair_base(I) + js) * 64),
                    (__attribute__((address_space(3))) void *)&cbs.CB[W][k ? N0 + js : js][0], 16, 0,
                    0);
        }
        asm volatile("" ::: "memory");
    };

    // ---- staging into LDS (phase B) ----
    // x and (x w) fragments of slab W, from xr: fragment s holds column 4m + s
    // of the 8 slots; w = dt exp2(G_last - G) per slot; x w is rounded once to
    // fp16.  G, dt and the column factor V = exp2(G_a - G) dt (a = the last
    // token of the 16-block) of the slab's 32 tokens go to G / DT / V (lanes
    // m = 0 write their 8 tokens).
    auto stage = [&]() {
        const float gs[8] = {gq[0].x, gq[0].y, gq[0].z, gq[0].w, gq[1].x, gq[1].y, gq[1].z, gq[1].w};
        const float ds[8] = {dq[0].x, dq[0].y, dq[0].z, dq[0].w, dq[1].x, dq[1].y, dq[1].z, dq[1].w};
        float wv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[e] = ds[e] * fast_exp2(glx - gs[e]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 xv, hv;
            uint32_t *xw = reinterpret_cast<uint32_t *>(&xv);
            uint32_t *hw = reinterpret_cast<uint32_t *>(&hv);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const uint32_t a0 = (s < 2) ? xr[2 * rr].x : xr[2 * rr].y;
                const uint32_t a1 = (s < 2) ? xr[2 * rr + 1].x : xr[2 * rr + 1].y;
                xw[rr] = (s & 1) ? pair_hi(a0, a1) : pair_lo(a0, a1);
                hw[rr] = pack_f16x2(bf16_lo(xw[rr]) * wv[2 * rr], bf16_hi(xw[rr]) * wv[2 * rr + 1]);
            }
            sm.XF[W][s][lane] = xv;
            sm.AF[W][s][lane] = hv;
        }
        // G at the last token of each 16-block of the slab (lane q = 3 holds it)
        const float ga0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gq[0].w), 48));
        const float ga1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gq[1].w), 48));
        if (m == 0) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int t = 32 * W + 16 * u + 4 * q;
                const float ga = u ? ga1 : ga0;
                const float4 gv = gq[u], dv = dq[u];
                *reinterpret_cast<float4 *>(&sm.G[t]) = gv;
                *reinterpret_cast<float4 *>(&sm.DT[t]) = dv;
                *reinterpret_cast<float4 *>(&sm.V[t]) =
                    make_float4(fast_exp2(ga - gv.x) * dv.x, fast_exp2(ga - gv.y) * dv.y,
                                fast_exp2(ga - gv.z) * dv.z, fast_exp2(ga - gv.w) * dv.w);
            }
        }
    };
    // the state as the B operand of the next inter product, in bf16:
    // element (p, n) goes to HF[n / 32][p % 4], lane (p / 4, (n % 32) / 8), slot n % 8
    auto stage_h = [&]() {
        uint16_t *hf = reinterpret_cast<uint16_t *>(&sm.HF[0][0][0]);
        const int kn = ncol >> 5, qq = (ncol >> 3) & 3, ee = ncol & 7;
#pragma unroll
        for (int i = 0; i < SPW; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int idx = (((kn * 4 + S0 + i) * 64) + qq * 16 + 4 * q + e) * 8 + ee;
                if constexpr (NTW == 2)
                    *reinterpret_cast<uint32_t *>(hf + idx) = pack_bf16x2(accs[i][0][e], accs[i][1][e]);
                else
                    *reinterpret_cast<uint2 *>(hf + idx) =
                        make_uint2(pack_bf16x2(accs[i][0][e], accs[i][1][e]),
                                   pack_bf16x2(accs[i][2][e], accs[i][3][e]));
            }
    };

    // ---- prologue: chunk 0 staged, its operands in flight ----
    // Load order (the vector-memory counter retires in order, so each wait
    // also covers everything issued before it): a chunk's tile pairs and C
    // fragments near the end of the previous chunk, its B fragments R slabs
    // ahead through a ring that runs on into the next chunk, the next x
    // mid-chunk.
    load_x(0);
    load_cb(0);
    load_c(0);
#pragma unroll
    for (int js = 0; js < R; ++js) load_b(0, js);
    stage();
    stage_h();
    lds_barrier();

    for (int32_t c = 0; c < a.nc; ++c) {
        {
            int t = threadIdx.x;
            asm volatile("" : "+v"(t));
            lane = t & 63;
            m = lane & 15;
            q = lane >> 4;
            ncol = 64 * (NT0 >> 2) + 4 * m + (NT0 & 3);
        }
        const int32_t nvalid = nvalid_of(c);
        const int64_t t0 = (int64_t)c * L;
        // ======== phase A: chunk c from the LDS buffers ========
        const float dec = fast_exp2(sm.G[L - 1]);
#pragma unroll
        for (int i = 0; i < SPW; ++i)
#pragma unroll
            for (int j = 0; j < NTW; ++j) accs[i][j] *= dec;

        // inter: accy[k][s][e] = y[16 I_k + 4q + e][4m + s] = C h^T, rows scaled by exp2(G)
        f32x4 accy[2][4];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int s = 0; s < 4; ++s) accy[k][s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kn = 0; kn < NK; ++kn)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 hfr = as_bf16x8(sm.HF[kn][s][lane]);
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    accy[k][s] = mfma16x16x32(as_bf16x8(cfr[k][kn]), hfr, accy[k][s]);
            }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int I = k ? I1 : I0;
            const float4 gi = *reinterpret_cast<const float4 *>(&sm.G[16 * I + 4 * q]);
            const float sc[4] = {fast_exp2(gi.x), fast_exp2(gi.y), fast_exp2(gi.z), fast_exp2(gi.w)};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e) accy[k][s][e] *= sc[e];
        }
        // this chunk's tile pairs have landed in LDS (the wait also covers the
        // previous chunk's y stores and the B fragments issued before them)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

        // the gate of this lane's outputs (rows 16 I + 4q + e, columns 4m..4m+3)
        uint2 zr[2][4];
        if constexpr (GATE) {
            const uint16_t *zb = a.z + ((b * a.T + t0) * a.H + h) * P + 4 * m;
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int il = 16 * (k ? I1 : I0) + 4 * q + e;
                    zr[k][e] = load_nt(zb + (int64_t)min(il, nvalid - 1) * XR);
                }
        }

        // per slab: the state product and the intra product
#pragma unroll
        for (int js = 0; js < NS; ++js) {
            f16x8 bcur[NTW];
#pragma unroll
            for (int j = 0; j < NTW; ++j) bcur[j] = bfr[js % R][j];
            if (js + R < NS) load_b(c, js + R);
            else load_b(c + 1, js + R - NS);
            if (js == XLOAD_AT) load_x(c + 1);
            // state: accs += (x w)^T B over the slab's 32 tokens (fp16 operands)
#pragma unroll
            for (int i = 0; i < SPW; ++i) {
                const f16x8 af = as_f16x8(sm.AF[js][S0 + i][lane]);
#pragma unroll
                for (int j = 0; j < NTW; ++j) accs[i][j] = mfma16x16x32(af, bcur[j], accs[i][j]);
            }
            // intra: the tile pairs of row blocks at or below this slab, drained
            bf16x8 xf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) xf[s] = as_bf16x8(sm.XF[js][s][lane]);
            const float4 vj0 = *reinterpret_cast<const float4 *>(&sm.V[32 * js + 4 * q]);
            const float4 vj1 = *reinterpret_cast<const float4 *>(&sm.V[32 * js + 16 + 4 * q]);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int I = k ? I1 : I0;
                if (I < 2 * js) continue;   // compile-time
                const float gi = sm.G[16 * I + m];    // this lane's output row i = 16 I + m
                const uint4 tp = cbs.CB[W][k ? N0 + js : js][lane];
                uint32_t cw[2][2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int J = 2 * js + u;
                    if (J > I) {
                        cw[u][0] = 0u;
                        cw[u][1] = 0u;
                        continue;
                    }
                    const uint32_t t0w = u ? tp.z : tp.x, t1w = u ? tp.w : tp.y;
                    const float ct[4] = {bf16_lo(t0w), bf16_hi(t0w), bf16_lo(t1w), bf16_hi(t1w)};
                    float v[4];
                    if (J < I) {
                        // exp2(G_i - G_j) dt_j = exp2(G_i - G_a) V_j, a = 16 J + 15
                        const float ui = fast_exp2(gi - sm.G[16 * J + 15]);
                        const float4 vj = u ? vj1 : vj0;
                        v[0] = ct[0] * (vj.x * ui);
                        v[1] = ct[1] * (vj.y * ui);
                        v[2] = ct[2] * (vj.z * ui);
                        v[3] = ct[3] * (vj.w * ui);
                    } else {
                        // diagonal block: exact pairwise decay, causal select (j <= i)
                        const float4 gj = *reinterpret_cast<const float4 *>(&sm.G[16 * J + 4 * q]);
                        const float4 dj = *reinterpret_cast<const float4 *>(&sm.DT[16 * J + 4 * q]);
                        const float gjv[4] = {gj.x, gj.y, gj.z, gj.w};
                        const float djv[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float val = ct[e] * fast_exp2(fminf(gi - gjv[e], 0.f)) * djv[e];
                            v[e] = (4 * q + e <= m) ? val : 0.f;
                        }
                    }
                    cw[u][0] = pack_bf16x2(v[0], v[1]);
                    cw[u][1] = pack_bf16x2(v[2], v[3]);
                }
                const bf16x8 af = as_bf16x8(make_uint4(cw[0][0], cw[0][1], cw[1][0], cw[1][1]));
#pragma unroll
                for (int s = 0; s < 4; ++s) accy[k][s] = mfma16x16x32(af, xf[s], accy[k][s]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // every tile pair of chunk c is drained: the next chunk's go into the
        // same slots; the next chunk's C fragments follow them
        load_cb(c + 1);
        load_c(c + 1);

        // ---- y = acc + D x (x from this lane's own fragments), fp32 or bf16 ----
        const int64_t yb = ((b * a.T + t0) * a.H + h) * P;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int I = k ? I1 : I0;
            // token 16 I + 4q + e sits in slot e + 4 (I & 1) of this lane's
            // fragment of slab I / 2: words (x, y) hold slots 0..3, (z, w) 4..7
            uint2 xw[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 f = sm.XF[I >> 1][s][lane];
                xw[s] = (I & 1) ? make_uint2(f.z, f.w) : make_uint2(f.x, f.y);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int il = 16 * I + 4 * q + e;
                if (il < nvalid) {
                    float o[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const uint32_t wd = (e < 2) ? xw[s].x : xw[s].y;
                        o[s] = accy[k][s][e] + Dh * ((e & 1) ? bf16_hi(wd) : bf16_lo(wd));
                    }
                    if constexpr (GATE) {   // y * silu(z)
                        const float zf[4] = {bf16_lo(zr[k][e].x), bf16_hi(zr[k][e].x),
                                             bf16_lo(zr[k][e].y), bf16_hi(zr[k][e].y)};
#pragma unroll
                        for (int s = 0; s < 4; ++s) o[s] *= fast_silu(zf[s]);
                    }
                    store_y4(a.y, yb + (int64_t)il * XR + 4 * m,
                             make_float4(o[0], o[1], o[2], o[3]), YBF);
                }
            }
        }
        lds_barrier();   // every read of chunk c's shared LDS buffers is done
        // ======== phase B: stage chunk c + 1 ========
        stage();
        stage_h();
        lds_barrier();
    }
    // nothing may still be writing this workgroup's LDS when it ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (a.fin) store_final();
}

template <int L, int N, bool GATE, bool YBF>
__global__ __launch_bounds__(64 * (L / 32), 1) void fused_fwd_kernel(FusedArgs a, uint32_t nblk) {
    __shared__ FusedSmem<L, N> sm;
    __shared__ FusedCbSmem<L> cbs;
    // logical id -> (b, h), heads fastest: a group's heads share an XCD's L2
    const uint32_t lid = xcd_remap(blockIdx.x, nblk);
    const int32_t h = (int32_t)(lid % (uint32_t)a.H);
    const int64_t b = lid / (uint32_t)a.H;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int NW = L / 32;
    switch (w) {
    case 0: fused_body<L, N, GATE, YBF, 0>(sm, cbs, a, b, h); break;
    case 1: fused_body<L, N, GATE, YBF, 1>(sm, cbs, a, b, h); break;
    case 2: if constexpr (NW > 2) fused_body<L, N, GATE, YBF, 2>(sm, cbs, a, b, h); break;
    case 3: if constexpr (NW > 2) fused_body<L, N, GATE, YBF, 3>(sm, cbs, a, b, h); break;
    case 4: if constexpr (NW > 4) fused_body<L, N, GATE, YBF, 4>(sm, cbs, a, b, h); break;
    case 5: if constexpr (NW > 4) fused_body<L, N, GATE, YBF, 5>(sm, cbs, a, b, h); break;
    case 6: if constexpr (NW > 4) fused_body<L, N, GATE, YBF, 6>(sm, cbs, a, b, h); break;
    default: if constexpr (NW > 4) fused_body<L, N, GATE, YBF, 7>(sm, cbs, a, b, h); break;
    }
}

template <int L, int N>
hipError_t launch_fused_ln(const Shape &s, const FusedArgs &a, hipStream_t st) {
    const uint64_t nblk = (uint64_t)s.Bt * s.H;
    // the gate and the output type are template parameters, as in chunk_scan
    const dim3 grid((uint32_t)nblk), blk(64 * (L / 32));
    if (a.z && s.ybf16)
        hipLaunchKernelGGL((fused_fwd_kernel<L, N, true, true>), grid, blk, 0, st, a, (uint32_t)nblk);
    else if (a.z)
        hipLaunchKernelGGL((fused_fwd_kernel<L, N, true, false>), grid, blk, 0, st, a, (uint32_t)nblk);
    else if (s.ybf16)
        hipLaunchKernelGGL((fused_fwd_kernel<L, N, false, true>), grid, blk, 0, st, a, (uint32_t)nblk);
    else
        hipLaunchKernelGGL((fused_fwd_kernel<L, N, false, false>), grid, blk, 0, st, a, (uint32_t)nblk);
    return hipGetLastError();
}

template <int L>
hipError_t launch_fused_l(const Shape &s, const FusedArgs &a, hipStream_t st) {
    if (s.N == 64) return launch_fused_ln<L, 64>(s, a, st);
    if (s.N == 128) return launch_fused_ln<L, 128>(s, a, st);
    return hipErrorInvalidValue;
}

}  // namespace

bool fused_fwd_supported(const Shape &s) {
    // bf16 io; per-chunk byte ranges of x and C rows fit the 32-bit buffer range
    const int64_t lim = (int64_t(1) << 31) - 1;
    return s.bf16 && s.P == 64 && s.L * s.H * s.P * 2 <= lim && s.L * s.G * s.N * 2 <= lim &&
           (uint64_t)s.Bt * s.H <= (uint64_t)lim;
}

size_t fused_cbt_bytes(const Shape &s) {
    return (size_t)s.Bt * s.nc * s.G * (size_t)cb_pair_base((int)(s.L / 16)) * 64 * 16;
}

hipError_t launch_fused_fwd(const Shape &s, const void *x, const void *C, const float *D,
                            const float *Gws, const float *DTws, const void *bfrag,
                            const void *cbt, const float *init, float *fin, void *y,
                            const void *z, hipStream_t st) {
    if (!fused_fwd_supported(s)) return hipErrorInvalidValue;
    if (s.Bt == 0 || s.H == 0) return hipSuccess;
    if (s.nc == 0 && !fin) return hipSuccess;
    FusedArgs a;
    a.x = (const uint16_t *)x;
    a.C = (const uint16_t *)C;
    a.z = (const uint16_t *)z;
    a.BF = (const uint4 *)bfrag;
    a.CBT = (const uint4 *)cbt;
    a.D = D;
    a.Gws = Gws;
    a.DTws = DTws;
    a.init = init;
    a.fin = fin;
    a.y = y;
    a.T = s.T;
    a.H = (int32_t)s.H;
    a.G = (int32_t)s.G;
    a.nc = (int32_t)s.nc;
    a.hpg = (int32_t)(s.H / s.G);
    switch (s.L) {
    case 64: return launch_fused_l<64>(s, a, st);
    case 128: return launch_fused_l<128>(s, a, st);
    case 256: return launch_fused_l<256>(s, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
