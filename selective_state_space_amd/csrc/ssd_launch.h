// Host-side launchers of the SSD kernels (internal to libssd.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// A validated problem shape.  P is always 64.
struct Shape {
    int64_t Bt, T, H, P, N, G, L, nc;  // nc = ceil(T / L)
    bool bf16;                          // io dtype: bf16 (else float32)
    bool ybf16;                         // y (y_t) stored as bf16 (bf16 io only), else float32
};

// dt_bias (NULL = none) and softplus: the optional dt preprocessing.  With
// bfrag non-NULL (bf16 B), the same launch also lays B out for launch_state_fwd
// (state_fwd_bfrag_bytes(s) bytes), which is then called with bfrag_ready.
hipError_t launch_chunk_cumsum(const Shape &s, const float *dt, const float *A, float *Gws,
                               float *DTws, const float *dt_bias, int softplus, hipStream_t st,
                               const void *B = nullptr, void *bfrag = nullptr);
hipError_t launch_chunk_state(const Shape &s, const void *x, const void *B, const float *Gws,
                              const float *DTws, float *S, hipStream_t st);
hipError_t launch_state_passing(const Shape &s, const float *S, const float *Gws,
                                const float *init, void *hprev, float *fin, hipStream_t st);
// z: output gate (x's dtype and layout), y <- y * silu(z); NULL = none.
hipError_t launch_chunk_scan(const Shape &s, const void *x, const void *B, const void *C,
                             const float *D, const float *Gws, const float *DTws,
                             const void *hprev, void *y, const void *z, hipStream_t st);
// chunk_state + state_passing in one pass (bf16 io).  rows_per_block = 4, 2
// or 1 row sets of the head per workgroup, 0 = chosen from the shape.
bool state_fwd_supported(const Shape &s);
bool state_fwd_preferred(const Shape &s);   // shape heuristic of the fused call
// bfrag: scratch of state_fwd_bfrag_bytes(s) bytes (B in fragment order).
size_t state_fwd_bfrag_bytes(const Shape &s);
hipError_t launch_state_fwd(const Shape &s, const void *x, const void *B, const float *Gws,
                            const float *DTws, const float *init, void *hprev, float *fin,
                            void *bfrag, int rows_per_block, bool hprev_f32, hipStream_t st,
                            bool bfrag_ready = false);
// The fused forward (bf16 io): launch_fused_prep runs the cumsum (G, DT), lays
// B out in the fused pass's fragment order (bfrag, state_fwd_bfrag_bytes(s))
// and forms the causal C B^T tiles (cbt, fused_cbt_bytes(s)), in one launch;
// launch_fused_fwd then carries the state through the chunks of every (b, h)
// and writes y (and the final state) in one pass.
bool fused_fwd_supported(const Shape &s);
size_t fused_cbt_bytes(const Shape &s);
hipError_t launch_fused_prep(const Shape &s, const float *dt, const float *A, float *Gws,
                             float *DTws, const float *dt_bias, int softplus, const void *B,
                             const void *C, void *bfrag, void *cbt, hipStream_t st);
hipError_t launch_fused_fwd(const Shape &s, const void *x, const void *C, const float *D,
                            const float *Gws, const float *DTws, const void *bfrag,
                            const void *cbt, const float *init, float *fin, void *y,
                            const void *z, hipStream_t st);
// The backward's adjoint scan in the same one-pass form, chunks last to
// first: ghat[c] (fp32, the adjoint of the state leaving chunk c) and dinit
// (NULL = not written) from dy (fp32), C (bf16) and dfinal (NULL = zero);
// cfrag: scratch of state_fwd_bfrag_bytes(s) bytes (C in fragment order).
bool state_adj_supported(const Shape &s);
int state_fwd_rows_per_block(const Shape &s);   // the row split chosen for a shape
int state_adj_rows_per_block(const Shape &s);
hipError_t launch_state_adj(const Shape &s, const float *dy, const void *C, const float *Gws,
                            const float *dfinal, float *ghat, float *dinit, void *cfrag,
                            int rows_per_block, hipStream_t st);
// Both one-pass scans of the backward in one grid (the same row split for
// both): the h_prev (fp32) and final-state recompute from x and the B
// fragments already in bfrag, and the adjoint scan of launch_state_adj (C
// laid out into cfrag first).
hipError_t launch_state_pair(const Shape &s, const void *x, const float *Gws, const float *DTws,
                             const float *init, float *hprev32, float *fin, const void *bfrag,
                             const float *dy, const void *C, const float *dfinal, float *ghat,
                             float *dinit, void *cfrag, int rows_per_block, hipStream_t st);
// K = s.T tokens per sequence; snaps / parent NULL = none; update = 0 leaves
// the state unwritten.
struct MultiArgs {
    float *state;
    const void *x;
    const float *dt;
    const void *B, *C;
    const float *A, *D;
    void *y;
    const float *dt_bias;
    int softplus;
    const void *z;
    float *snaps;
    const int32_t *parent;
    int update;
};
hipError_t launch_decode_multi(const Shape &s, const MultiArgs &m, hipStream_t st);
// The decode step on a 16-bit state (fp16 nearest or stochastic, bf16, or
// int16 codes with per-row decode scales in `scale`).
enum LowpFormat { LOWP_F16 = 1, LOWP_BF16 = 2, LOWP_INT16 = 3 };
struct LowpArgs {
    void *state;
    float *scale;
    int format;
    int philox_rounds;   // fp16: > 0 = stochastic rounding with that many rounds
    uint64_t seed;
    const void *x;
    const float *dt;
    const void *B, *C;
    const float *A, *D;
    void *y;
    const float *dt_bias;
    int softplus;
    const void *z;
};
hipError_t launch_decode_lowp(const Shape &s, const LowpArgs &a, hipStream_t st);

// The backward of the chunked forward.  G, DT, hprev and fin come from the
// forward stages run again on the same workspace; S (the forward's S region,
// dead by then) receives the chunk adjoints; CB (fp32 io) or CB3/CBT3 (bf16
// io), MT, tok (3 planes of Bt*H*nc*L floats) and part (3 * Bt*H doubles) are
// backward scratch.
struct BwdArgs {
    const void *x, *B, *C;
    const float *A, *D, *dy, *dfinal, *fin;
    float *dinit, *dx, *ddt, *dA, *dB, *dC, *dD;
    const float *G, *DT;
    float *S;
    const void *hprev;
    float *CB, *tok;         // CB: C B^T in fp32, fp32 io only (NULL otherwise)
    uint16_t *CB3, *CBT3;    // C B^T and its transpose as three bf16 terms each, bf16 io only
    float *MT;               // the dB/dC matrix M, transposed, bf16 io only
    double *part;
    bool ghat_ready;         // S already holds ghat and dinit is written (launch_state_adj)
};
size_t bwd_cb_bytes(const Shape &s);
hipError_t launch_chunked_bwd(const Shape &s, const BwdArgs &a, hipStream_t st);
hipError_t launch_decode_step(const Shape &s, float *state, const void *x, const float *dt,
                              const void *B, const void *C, const float *A, const float *D,
                              void *y, const float *dt_bias, int softplus, const void *z,
                              hipStream_t st);

}  // namespace ssd
