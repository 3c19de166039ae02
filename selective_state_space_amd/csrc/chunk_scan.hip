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
// bf16 path (MFMA, v_mfma_f32_16x16x32_bf16): one workgroup per (b, chunk,
// group, block of heads), heads of the block processed in turn.  C B^T depends
// only on the group, so it is formed once per workgroup and reused by every
// head: the chunk's B and C are staged in LDS as MFMA fragments (16 bytes per
// lane, lane-linear: every operand read is one conflict-free ds_read_b128),
// and each wavefront computes the causal 16x16 tiles of its row blocks --
// paired (I, L/16-1-I) so every wavefront holds the same number of tiles --
// and keeps them in registers as packed bf16 for all heads.  Row-block
// ownership is a template parameter (the wavefront index is dispatched once),
// so every tile index is a compile-time register index.
// Per head (its x^T fragments, h_prev fragments, G, dt and column factors V
// staged in LDS; the next head's loads are in flight while this one runs):
//   1. inter: acc = C h_prev^T (K = N); output column m of MFMA s is p = 4m+s.
//      Rows are then scaled by exp2(G_i).
//   2. intra: each cached tile (C B^T)^T (lane m: column i, rows j = 4q..4q+3)
//      is a 4-element K slice of the A operand for row i, so the drain --
//      times exp2(G_i - G_j) dt_j, select j <= i, round to bf16 -- produces the
//      A operand of the second product in registers, with no LDS round trip.
//      Below the diagonal the decay factors through the last token a of the
//      column block: exp2(G_i - G_j) = exp2(G_i - G_a) * exp2(G_a - G_j), both
//      exponents <= 0, so a tile needs one exp2 per lane (V_j = exp2(G_a - G_j)
//      dt_j is staged per token).  Diagonal tiles use the exact pairwise
//      exponent with a causal select.  Tiles above the diagonal do not exist.
//   3. y = acc + D x (x from the lane's own fragment), written fp32 (or bf16
//      when the caller asks for y in the io dtype).
//
// fp32 path (VALU): one workgroup per (b, h, chunk), 16-row tiles: the
// decayed, masked C B^T rows are built in LDS, then each thread forms y for
// one p and four rows.

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

// Wavefronts per workgroup: 8 for 256-token chunks (each owns one row-block
// pair), 4 otherwise.
template <int L>
struct ScanWaves {
    static constexpr int NW = L == 256 ? 8 : 4;
};

// Row blocks (16 rows each) owned by wavefront W of NW, paired (I, NB-1-I) so
// that every wavefront holds the same number of causal tiles (NB + 1 per pair).
template <int NB, int NW, int W>
struct RowBlocks {
    static constexpr int RBW = NB >= 2 * NW ? NB / NW : 1;
    static constexpr int at(int k) {
        // NB == 2 NW: one pair per wavefront; NB == 4 NW: two pairs; NB == NW: one block
        return NB == NW ? W
                        : (NB == 2 * NW ? (k == 0 ? W : NB - 1 - W)
                                        : (k == 0 ? W : k == 1 ? NB - 1 - W
                                                        : k == 2 ? W + NW : NB - 1 - NW - W));
    }
    static constexpr int tiles_before(int k) {
        int t = 0;
        for (int i = 0; i < k; ++i) t += at(i) + 1;
        return t;
    }
    static constexpr int ntiles = tiles_before(RBW);
};

// LDS of one workgroup: first the chunk's B as MFMA fragments (to form the
// C B^T tiles once), then -- reusing the same bytes -- two buffers of per-head
// data, every operand in fragment order (16 bytes per lane, lane-linear), so
// each operand read is one conflict-free ds_read_b128 at a constant offset.
template <int L, int N>
struct ScanSmem {
    static constexpr int NK = N / 32, NS = L / 32, NB = L / 16;
    struct Head {
        uint4 XF[NS][4][64];  // x^T fragments: slab js, p = 4m + s
        uint4 HF[NK][4][64];  // h_prev fragments: n-step kn, p = 4m + s
        float G[L], V[L], DT[L];
    };
    uint4 CF[NB][NK][64];      // C fragments: 16-token block I, n-step kn (whole workgroup life)
    union {
        uint4 BF[NB][NK][64];  // B fragments (C B^T phase only)
        Head hd;               // the head being computed
    };
};

template <int L, int N>
struct ScanArgs {
    const uint16_t *x, *Bm, *Cm, *hprev;
    const uint16_t *z;   // output gate (GATE instantiations only)
    const float *D, *Gws, *DTws;
    void *y;             // float32, or bf16 in the YBF instantiations
    int64_t T;
    int32_t H, G, nc, hpg, NH, nhb;
};

// Everything one head of the workgroup needs, loaded into registers (issued
// one head ahead of use) and then written to an LDS head buffer.
template <int L, int N>
struct HeadRegs {
    static constexpr int NS = L / 32, NK = N / 32, NW = ScanWaves<L>::NW;
    static constexpr int XSW = (NS + NW - 1) / NW;
    static constexpr int HPL = (NK * 4 + NW - 1) / NW;
    uint2 xr[XSW][8];
    uint4 hv[HPL];
    float g, gl, dt, dh;   // G, G at the end of the token's 16-block, dt; D of the head
};

template <int L, int N, bool RAGGED>
__device__ __forceinline__ void head_load(HeadRegs<L, N> &r, const ScanArgs<L, N> &a, int64_t b,
                                          int32_t h, int32_t c, int32_t nvalid, int w, int lane) {
    constexpr int P = 64, NS = L / 32, NK = N / 32, NW = ScanWaves<L>::NW;
    const int m = lane & 15, q = lane >> 4, tid = 64 * w + lane;
    const int64_t t0 = (int64_t)c * L;
    const uint16_t *xb = a.x + ((b * a.T + t0) * a.H + h) * P;
    const int32_t XR = a.H * P;
#pragma unroll
    for (int k = 0; k < HeadRegs<L, N>::XSW; ++k) {
        const int js = w + NW * k;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int tl = 32 * js + ((rr < 4) ? 0 : 16) + 4 * q + (rr & 3);
            r.xr[k][rr] = (js < NS && (!RAGGED || tl < nvalid))
                              ? load_nt(xb + tl * XR + 4 * m)
                              : make_uint2(0u, 0u);
        }
    }
    const int64_t bhc = ((int64_t)b * a.H + h) * a.nc + c;
    const uint16_t *hp = a.hprev + bhc * (int64_t)(P * N);
#pragma unroll
    for (int k = 0; k < HeadRegs<L, N>::HPL; ++k) {
        const int pc = w + NW * k, kn = pc >> 2, s = pc & 3;
        r.hv[k] = (pc < NK * 4)
                      ? *reinterpret_cast<const uint4 *>(hp + (4 * m + s) * N + 32 * kn + 8 * q)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
    // Unconditional (threads past L load token L-1 again): a load under a
    // branch, or one used right after issue, makes the compiler wait with
    // vmcnt(0), which would drain this prefetch as well.
    const int tk = tid < L ? tid : L - 1;
    const float *Gp = a.Gws + bhc * L;
    r.g = Gp[tk];
    r.gl = Gp[tk | 15];
    r.dt = a.DTws[bhc * L + tk];
    r.dh = a.D[h];
}

template <int L, int N>
__device__ __forceinline__ void head_store(typename ScanSmem<L, N>::Head &hd,
                                           const HeadRegs<L, N> &r, int w, int lane) {
    constexpr int NS = L / 32, NK = N / 32, NW = ScanWaves<L>::NW;
    const int tid = 64 * w + lane;
#pragma unroll
    for (int k = 0; k < HeadRegs<L, N>::XSW; ++k) {
        const int js = w + NW * k;
        if (js < NS) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint4 v;
                uint32_t *vw = reinterpret_cast<uint32_t *>(&v);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const uint32_t a0 = (s < 2) ? r.xr[k][2 * rr].x : r.xr[k][2 * rr].y;
                    const uint32_t a1 = (s < 2) ? r.xr[k][2 * rr + 1].x : r.xr[k][2 * rr + 1].y;
                    vw[rr] = (s & 1) ? pair_hi(a0, a1) : pair_lo(a0, a1);
                }
                hd.XF[js][s][lane] = v;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < HeadRegs<L, N>::HPL; ++k) {
        const int pc = w + NW * k;
        if (pc < NK * 4) hd.HF[pc >> 2][pc & 3][lane] = r.hv[k];
    }
    if (tid < L) {
        // V_j = exp2(G_a - G_j) dt_j, a = the last token of j's 16-block
        // (exponent <= 0): the column factor of the decay between blocks.
        hd.G[tid] = r.g;
        hd.DT[tid] = r.dt;
        hd.V[tid] = fast_exp2(r.gl - r.g) * r.dt;
    }
}

template <int L, int N, bool RAGGED, bool GATE, bool YBF, int W>
__device__ __forceinline__ void chunk_scan_group(ScanSmem<L, N> &sm, const ScanArgs<L, N> &a,
                                                 int64_t b, int32_t c, int32_t g, int32_t h0,
                                                 int32_t nh, int32_t nvalid) {
    constexpr int P = 64;
    constexpr int NB = L / 16, NK = N / 32, NS = L / 32, NW = ScanWaves<L>::NW;
    using RB = RowBlocks<NB, NW, W>;
    constexpr int RBW = RB::RBW;
    constexpr int NT = RB::ntiles;
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, q = lane >> 4, tid = threadIdx.x;
    const int64_t t0 = (int64_t)c * L;
    const uint16_t *bb = a.Bm + ((b * a.T + t0) * a.G + g) * N;
    const uint16_t *cb = a.Cm + ((b * a.T + t0) * a.G + g) * N;
    const int32_t BR = a.G * N;
    auto valid = [&](int tl) { return !RAGGED || tl < nvalid; };

    // ---- the group's C B^T tiles, once for all heads of the workgroup ----
    HeadRegs<L, N> pre;
    head_load<L, N, RAGGED>(pre, a, b, h0, c, nvalid, W, lane);   // first head, in flight now
    {
        constexpr int PPT = NB * NK / NW;   // B (and C) pieces per thread
        uint4 bv[PPT], cv[PPT];
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int pc = W + NW * k, J = pc / NK, kn = pc % NK;
            const int tl = 16 * J + m;
            const int off = tl * BR + 32 * kn + 8 * q;
            bv[k] = valid(tl) ? *reinterpret_cast<const uint4 *>(bb + off) : make_uint4(0u, 0u, 0u, 0u);
            cv[k] = valid(tl) ? *reinterpret_cast<const uint4 *>(cb + off) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int pc = W + NW * k;
            sm.BF[pc / NK][pc % NK][lane] = bv[k];
            sm.CF[pc / NK][pc % NK][lane] = cv[k];
        }
    }
    lds_barrier();
    // (C B^T)^T tiles, kept for all heads as packed bf16: tile t, element e =
    // C_i . B_j with i = 16I + m, j = 16J + 4q + e (words: e = 0,1 | 2,3)
    uint2 cbt[NT];
#pragma unroll
    for (int k = 0; k < RBW; ++k) {
#pragma unroll
        for (int J = 0; J <= RB::at(k); ++J) {
            f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kn = 0; kn < NK; ++kn)
                t = mfma16x16x32(as_bf16x8(sm.BF[J][kn][lane]), as_bf16x8(sm.CF[RB::at(k)][kn][lane]), t);
            cbt[RB::tiles_before(k) + J] = make_uint2(pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3]));
            // two tiles' MFMA chains in flight at a time (bounded register life)
            if (J & 1) __builtin_amdgcn_sched_barrier(0);
        }
    }
    lds_barrier();   // BF is dead; the head buffer takes its place
    head_store<L, N>(sm.hd, pre, W, lane);
    float dh = pre.dh;   // D of the head being computed (pre is refilled ahead)
    lds_barrier();

    for (int hh = 0; hh < nh; ++hh) {
        const int h = h0 + hh;
        auto &hd = sm.hd;
        // the next head's operands, unconditionally (the last head reloads
        // itself) and pinned here: under a branch the compiler sinks these
        // loads down to their use and nothing is left in flight
        head_load<L, N, RAGGED>(pre, a, b, min(h + 1, h0 + nh - 1), c, nvalid, W, lane);
        __builtin_amdgcn_sched_barrier(0);

        // ---- inter: acc = C h_prev^T, rows scaled by exp2(G_i) ----
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
                const bf16x8 hf = as_bf16x8(hd.HF[kn][s][lane]);
#pragma unroll
                for (int k = 0; k < RBW; ++k)
                    acc[k][s] = mfma16x16x32(as_bf16x8(sm.CF[RB::at(k)][kn][lane]), hf, acc[k][s]);
            }
#pragma unroll
        for (int k = 0; k < RBW; ++k) {
            const float4 gi = *reinterpret_cast<const float4 *>(&hd.G[16 * RB::at(k) + 4 * q]);
            const float sc[4] = {fast_exp2(gi.x), fast_exp2(gi.y), fast_exp2(gi.z),
                                 fast_exp2(gi.w)};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[k][s][e] *= sc[e];
        }

        // the gate of this lane's outputs (rows 16 I + 4q + e, columns 4m..4m+3),
        // loaded two slabs before the end of the intra products and used in
        // the epilogue: issued any earlier, its registers push the products
        // into spills
        constexpr int kZLead = 2;
        uint2 zr[RBW][4];
        auto load_z = [&]() {
            const uint16_t *zb = a.z + ((b * a.T + t0) * a.H + h) * P + 4 * m;
#pragma unroll
            for (int k = 0; k < RBW; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int il = 16 * RB::at(k) + 4 * q + e;
                    const int ic = RAGGED ? min(il, nvalid - 1) : il;   // unconditional
                    zr[k][e] = load_nt(zb + (int64_t)ic * a.H * P);
                }
        };
        __builtin_amdgcn_sched_barrier(0);
        // ---- intra: the cached tiles drained with this head's decay ----
#pragma unroll
        for (int js = 0; js < NS; ++js) {
            if constexpr (GATE)
                if (js == (NS > kZLead ? NS - kZLead : 0)) load_z();
            bf16x8 xf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) xf[s] = as_bf16x8(hd.XF[js][s][lane]);
            const float4 vj0 = *reinterpret_cast<const float4 *>(&hd.V[32 * js + 4 * q]);
            const float4 vj1 = *reinterpret_cast<const float4 *>(&hd.V[32 * js + 16 + 4 * q]);
#pragma unroll
            for (int k = 0; k < RBW; ++k) {
                const int I = RB::at(k);
                if (I < 2 * js) continue;   // compile-time
                const float gi = hd.G[16 * I + m];    // this lane's output row i = 16I + m
                uint32_t cw[2][2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int J = 2 * js + u;
                    if (J > I) {
                        cw[u][0] = 0u;
                        cw[u][1] = 0u;
                        continue;
                    }
                    const uint2 cw2 = cbt[RB::tiles_before(k) + J];
                    const float ct[4] = {bf16_lo(cw2.x), bf16_hi(cw2.x), bf16_lo(cw2.y),
                                         bf16_hi(cw2.y)};
                    float v[4];
                    if (J < I) {
                        // exp2(G_i - G_j) dt_j = exp2(G_i - G_a) * V_j, a = 16J + 15
                        const float ui = fast_exp2(gi - hd.G[16 * J + 15]);
                        const float4 vj = u ? vj1 : vj0;
                        v[0] = ct[0] * (vj.x * ui);
                        v[1] = ct[1] * (vj.y * ui);
                        v[2] = ct[2] * (vj.z * ui);
                        v[3] = ct[3] * (vj.w * ui);
                    } else {
                        // diagonal block: exact pairwise decay, causal select (j <= i)
                        const float4 gj = *reinterpret_cast<const float4 *>(&hd.G[16 * J + 4 * q]);
                        const float4 dj = *reinterpret_cast<const float4 *>(&hd.DT[16 * J + 4 * q]);
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
                for (int s = 0; s < 4; ++s) acc[k][s] = mfma16x16x32(af, xf[s], acc[k][s]);
            }
            // keep each slab's LDS reads next to their use (bounded register life)
            __builtin_amdgcn_sched_barrier(0);
        }

        __builtin_amdgcn_sched_barrier(0);
        // ---- y = acc + D x (x from this lane's own fragments), fp32 or bf16 ----
        const float Dh = dh;
        const int64_t yb = ((b * a.T + t0) * a.H + h) * P;   // element offset of row 0
        const int32_t XR = a.H * P;
#pragma unroll
        for (int k = 0; k < RBW; ++k) {
            const int I = RB::at(k);
            // token 16I + 4q + e sits in K slot e + 4 (I & 1) of this lane's
            // fragment of slab I/2: words (x, y) hold slots 0..3, (z, w) 4..7
            uint2 xw[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 f = hd.XF[I >> 1][s][lane];
                xw[s] = (I & 1) ? make_uint2(f.z, f.w) : make_uint2(f.x, f.y);
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
                    float o[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) o[s] = acc[k][s][e] + Dh * xv[s];
                    if constexpr (GATE) {   // y * silu(z)
                        const float zf[4] = {bf16_lo(zr[k][e].x), bf16_hi(zr[k][e].x),
                                             bf16_lo(zr[k][e].y), bf16_hi(zr[k][e].y)};
#pragma unroll
                        for (int s = 0; s < 4; ++s) o[s] *= fast_silu(zf[s]);
                    }
                    store_y4(a.y, yb + il * XR + 4 * m, make_float4(o[0], o[1], o[2], o[3]), YBF);
                }
            }
        }
        if (hh + 1 < nh) {
            lds_barrier();   // every wavefront is done with this head's buffer
            head_store<L, N>(sm.hd, pre, W, lane);
            dh = pre.dh;
            lds_barrier();
        }
    }
}

template <int L, int N, bool RAGGED, bool GATE, bool YBF>
__device__ __forceinline__ void chunk_scan_dispatch(ScanSmem<L, N> &sm, const ScanArgs<L, N> &a,
                                                    int64_t b, int32_t c, int32_t g, int32_t h0,
                                                    int32_t nh, int32_t nvalid) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (ScanWaves<L>::NW == 8) {
        switch (w) {
        case 0: chunk_scan_group<L, N, RAGGED, GATE, YBF, 0>(sm, a, b, c, g, h0, nh, nvalid); break;
        case 1: chunk_scan_group<L, N, RAGGED, GATE, YBF, 1>(sm, a, b, c, g, h0, nh, nvalid); break;
        case 2: chunk_scan_group<L, N, RAGGED, GATE, YBF, 2>(sm, a, b, c, g, h0, nh, nvalid); break;
        case 3: chunk_scan_group<L, N, RAGGED, GATE, YBF, 3>(sm, a, b, c, g, h0, nh, nvalid); break;
        case 4: chunk_scan_group<L, N, RAGGED, GATE, YBF, 4>(sm, a, b, c, g, h0, nh, nvalid); break;
        case 5: chunk_scan_group<L, N, RAGGED, GATE, YBF, 5>(sm, a, b, c, g, h0, nh, nvalid); break;
        case 6: chunk_scan_group<L, N, RAGGED, GATE, YBF, 6>(sm, a, b, c, g, h0, nh, nvalid); break;
        default: chunk_scan_group<L, N, RAGGED, GATE, YBF, 7>(sm, a, b, c, g, h0, nh, nvalid); break;
        }
    } else {
        switch (w) {
        case 0: chunk_scan_group<L, N, RAGGED, GATE, YBF, 0>(sm, a, b, c, g, h0, nh, nvalid); break;
        case 1: chunk_scan_group<L, N, RAGGED, GATE, YBF, 1>(sm, a, b, c, g, h0, nh, nvalid); break;
        case 2: chunk_scan_group<L, N, RAGGED, GATE, YBF, 2>(sm, a, b, c, g, h0, nh, nvalid); break;
        default: chunk_scan_group<L, N, RAGGED, GATE, YBF, 3>(sm, a, b, c, g, h0, nh, nvalid); break;
        }
    }
}

template <int L, int N, bool GATE, bool YBF>
__global__ __launch_bounds__(64 * ScanWaves<L>::NW, 1) void chunk_scan_bf16_kernel(
    ScanArgs<L, N> a, uint32_t nblk) {
    __shared__ ScanSmem<L, N> sm;
    // logical id -> (b, chunk, group, head block), head blocks fastest
    const uint32_t lid = xcd_remap(blockIdx.x, nblk);
    const int32_t hb = lid % a.nhb;
    const uint32_t rest = lid / a.nhb;
    const int32_t g = rest % a.G;
    const int32_t c = (rest / a.G) % a.nc;
    const int64_t b = rest / ((uint32_t)a.G * a.nc);
    const int32_t h0 = g * a.hpg + hb * a.NH;
    const int32_t nh = min(a.NH, a.hpg - hb * a.NH);
    const int64_t rem = a.T - (int64_t)c * L;
    const int32_t nvalid = rem < L ? (int32_t)rem : L;
    if (nvalid == L)
        chunk_scan_dispatch<L, N, false, GATE, YBF>(sm, a, b, c, g, h0, nh, nvalid);
    else
        chunk_scan_dispatch<L, N, true, GATE, YBF>(sm, a, b, c, g, h0, nh, nvalid);
}

template <int L, int N>
__global__ __launch_bounds__(256) void chunk_scan_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ Bm, const float *__restrict__ Cm,
    const float *__restrict__ D, const float *__restrict__ Gws, const float *__restrict__ DTws,
    const float *__restrict__ hprev, float *__restrict__ y, const float *__restrict__ z,
    int64_t T, int32_t H, int32_t G, int32_t nc, uint32_t nblk) {
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
            float out = acc + Dh * x[off];
            if (z) out *= fast_silu(z[off]);   // y * silu(z)
            y[off] = out;
        }
    }
}

// Heads per workgroup: enough heads share one set of C B^T tiles to amortise
// them, while the grid is one round of resident workgroups: about 256 (one
// per CU) at L = 256, whose 128 KB of LDS allows one per CU, else 512.
inline int32_t heads_per_block(const Shape &s) {
    const int64_t hpg = s.H / s.G;
    const int64_t groups = s.Bt * s.nc * s.G;
    const int64_t slots = s.L == 256 ? 256 : 512;
    int64_t nh = (groups * hpg + slots - 1) / slots;
    if (nh < 1) nh = 1;
    if (nh > hpg) nh = hpg;
    return (int32_t)nh;
}

template <int L, int N>
hipError_t launch_scan(const Shape &s, const void *x, const void *B, const void *C,
                       const float *D, const float *Gws, const float *DTws, const void *hprev,
                       void *y, const void *z, hipStream_t st) {
    if (s.bf16) {
        ScanArgs<L, N> a;
        a.x = (const uint16_t *)x;
        a.z = (const uint16_t *)z;
        a.Bm = (const uint16_t *)B;
        a.Cm = (const uint16_t *)C;
        a.hprev = (const uint16_t *)hprev;
        a.D = D;
        a.Gws = Gws;
        a.DTws = DTws;
        a.y = y;
        a.T = s.T;
        a.H = (int32_t)s.H;
        a.G = (int32_t)s.G;
        a.nc = (int32_t)s.nc;
        a.hpg = (int32_t)(s.H / s.G);
        a.NH = heads_per_block(s);
        a.nhb = (a.hpg + a.NH - 1) / a.NH;
        const uint64_t nblk = (uint64_t)s.Bt * s.nc * s.G * a.nhb;
        // the gate and the output type are template parameters: no per-element
        // branch in the epilogue, and each variant carries its own kernel name
        const dim3 grid((uint32_t)nblk), blk(64 * ScanWaves<L>::NW);
        if (z && s.ybf16)
            hipLaunchKernelGGL((chunk_scan_bf16_kernel<L, N, true, true>), grid, blk, 0, st, a, (uint32_t)nblk);
        else if (z)
            hipLaunchKernelGGL((chunk_scan_bf16_kernel<L, N, true, false>), grid, blk, 0, st, a, (uint32_t)nblk);
        else if (s.ybf16)
            hipLaunchKernelGGL((chunk_scan_bf16_kernel<L, N, false, true>), grid, blk, 0, st, a, (uint32_t)nblk);
        else
            hipLaunchKernelGGL((chunk_scan_bf16_kernel<L, N, false, false>), grid, blk, 0, st, a, (uint32_t)nblk);
    } else {
        const uint64_t nblk = (uint64_t)s.Bt * s.nc * s.H;
        hipLaunchKernelGGL((chunk_scan_f32_kernel<L, N>), dim3((uint32_t)nblk), dim3(256), 0, st,
                           (const float *)x, (const float *)B, (const float *)C, D, Gws, DTws,
                           (const float *)hprev, (float *)y, (const float *)z, s.T,
                           (int32_t)s.H, (int32_t)s.G, (int32_t)s.nc, (uint32_t)nblk);
    }
    return hipGetLastError();
}

template <int L>
hipError_t launch_scan_n(const Shape &s, const void *x, const void *B, const void *C,
                         const float *D, const float *Gws, const float *DTws, const void *hprev,
                         void *y, const void *z, hipStream_t st) {
    if (s.N == 64) return launch_scan<L, 64>(s, x, B, C, D, Gws, DTws, hprev, y, z, st);
    if (s.N == 128) return launch_scan<L, 128>(s, x, B, C, D, Gws, DTws, hprev, y, z, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_scan(const Shape &s, const void *x, const void *B, const void *C,
                             const float *D, const float *Gws, const float *DTws,
                             const void *hprev, void *y, const void *z, hipStream_t st) {
    if (s.Bt == 0 || s.nc == 0) return hipSuccess;
    switch (s.L) {
    case 64: return launch_scan_n<64>(s, x, B, C, D, Gws, DTws, hprev, y, z, st);
    case 128: return launch_scan_n<128>(s, x, B, C, D, Gws, DTws, hprev, y, z, st);
    case 256: return launch_scan_n<256>(s, x, B, C, D, Gws, DTws, hprev, y, z, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
