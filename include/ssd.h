/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 SSD layer scan library
 * (libssd.so).
 *
 * The layer ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels
 * in NVIDIA CUDA Tile", section "Mamba-2 architecture"; "Optimizing Nemotron
 * v3 Super in TensorRT-LLM", section 6.1 "The SSU Math"), per batch row b and
 * head h, with g = h / (H / G) the head's group:
 *
 *     h_t = exp(A_h dt_t) h_{t-1} + dt_t x_t (outer) B_t     state [P][N]
 *     y_t = h_t C_t + D_h x_t                                 output [P]
 *
 * The output uses the updated state h_t.  The forward computes this chunk by
 * chunk (the SSD form of the same page, sections "Kernel 1" to "Kernel 3"):
 *
 *   chunk_cumsum   G = log2(e) * chunk-local inclusive cumsum of A dt
 *   chunk_state    S_c = sum_j exp2(G_last - G_j) dt_j x_j (outer) B_j
 *   state_passing  h_prev[c] = h;  h <- exp2(G_last) h + S_c
 *   chunk_scan     y = exp2(G) C h_prev^T
 *                      + (exp2(G_i - G_j) (C B^T)_ij dt_j [j <= i]) X + D X
 *
 * CONVENTIONS (every entry point)
 *   - All tensors are dense, contiguous, row-major, in DEVICE memory owned by
 *     the caller.  The library never allocates, frees or synchronizes.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns at once.
 *   - Arguments are validated on the host before any HIP call.  On a
 *     validation error nothing is launched or written, and
 *     ssd_last_error_detail() names the field and value.
 *   - Sizes and offsets are 64-bit throughout.
 *   - Unchecked preconditions: A <= 0, dt >= 0, all inputs finite.
 *   - Supported instantiation: headdim P = 64; dstate N in {64, 128};
 *     chunk_size L in {64, 128, 256}; io dtype SSD_F32 or SSD_BF16.
 *     batch and seqlen may be 0 (nothing to compute).
 *   - Every pointer must be 16-byte aligned.
 *   - Results are deterministic: no floating-point atomics; reruns are
 *     bitwise identical.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = -1,         /* a required pointer is NULL */
    SSD_ERR_SHAPE = -2,        /* a dimension is out of range, or H % G != 0 */
    SSD_ERR_UNSUPPORTED = -3,  /* P, N, chunk_size or dtype not instantiated */
    SSD_ERR_ALIGN = -4,        /* a pointer is not 16-byte aligned */
    SSD_ERR_WORKSPACE = -5,    /* workspace smaller than the queried size */
    SSD_ERR_HIP = -6           /* a HIP launch reported an error */
} ssd_status;

/* Element type of the inputs x, B, C (and x_t, B_t, C_t).  dt, A, D and every
 * state are always float32.  The outputs y and y_t are float32 by default:
 * stored in bf16, y carries its own rounding of up to 2^-8 |y|, which alone
 * exceeds 2e-2 rms(y) wherever |y| > 5 rms(y) -- and the D x skip term makes
 * such outputs common.  ssd_layer_opts.y_io_dtype stores them in the io dtype
 * instead (the pages' interfaces return y in x's dtype). */
typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef struct {
    int64_t batch;     /* Bt >= 0 */
    int64_t seqlen;    /* T >= 0 (ignored by the decode step) */
    int64_t nheads;    /* H >= 1 */
    int64_t headdim;   /* P, must be 64 */
    int64_t dstate;    /* N, 64 or 128 */
    int64_t ngroups;   /* G >= 1, H % G == 0; head h uses group h / (H / G) */
    int32_t io_dtype;  /* an ssd_dtype */
} ssd_dims;

/*
 * Chunked forward (the whole hot path: the four stages below, in order, on
 * `stream`).
 *
 *   x           [Bt, T, H, P]  io dtype      in
 *   dt          [Bt, T, H]     float32       in   (after any softplus)
 *   A, D        [H]            float32       in   (A natural-log decay rate)
 *   B, C        [Bt, T, G, N]  io dtype      in
 *   chunk_size  L in {64, 128, 256}
 *   init_state  [Bt, H, P, N]  float32       in   NULL = zeros
 *   y           [Bt, T, H, P]  float32       out  (io dtype with opts->y_io_dtype)
 *   final_state [Bt, H, P, N]  float32       out  NULL = not written
 *   workspace   ssd_chunked_fwd_workspace_size() bytes of device memory
 *
 * With batch or seqlen 0 the token tensors (x, dt, B, C, y) are empty and may
 * be NULL; with seqlen 0 final_state receives init_state (or zeros).
 *
 * init_state may equal final_state (in-place continuation: a sequence split
 * at a chunk boundary and run in two calls gives the state of one call);
 * any other overlap between arguments is undefined.  T need not be a
 * multiple of L: a ragged last chunk is computed as if padded with dt = 0.
 */
ssd_status ssd_chunked_fwd(const void *x, const float *dt, const float *A, const void *B,
                           const void *C, const float *D, int64_t chunk_size,
                           const float *init_state, void *y, float *final_state,
                           const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Bytes of device workspace ssd_chunked_fwd and the stage calls need
 * (0 for an invalid or empty shape). */
size_t ssd_chunked_fwd_workspace_size(const ssd_dims *dims, int64_t chunk_size);

/*
 * Byte offsets of the four workspace regions, so that tests can read the
 * intermediates.  With nc = ceil(T / L):
 *   offsets[0]  G       float32 [Bt, H, nc, L]   log2(e) * chunk-local cumsum of A dt
 *   offsets[1]  DT      float32 [Bt, H, nc, L]   dt transposed, 0 past T
 *   offsets[2]  S       float32 [Bt, H, nc, P, N] per-chunk states (four-stage
 *               path); on the other paths it holds B re-laid out in MFMA
 *               fragment order instead (contents unspecified)
 *   offsets[3]  h_prev  io dtype [Bt, H, nc, P, N] state entering each chunk
 *               (bf16 for bf16 inputs: it is an MFMA operand of chunk_scan);
 *               unspecified after a call on the fused path
 * Each region starts on a 256-byte boundary.
 */
ssd_status ssd_chunked_fwd_workspace_layout(const ssd_dims *dims, int64_t chunk_size,
                                            size_t offsets[4]);

/*
 * The four stages of the chunked forward, callable one at a time (same
 * arguments and workspace; each reads what the previous stage left in the
 * workspace): chunk_cumsum, chunk_state, state_passing, chunk_scan in this
 * order give y, final_state and every intermediate.  ssd_chunked_fwd takes
 * one of three paths (ssd_chunked_fwd_path says which): the four stages
 * (fp32 io), chunk_cumsum + the one-pass ssd_state_fwd stage + chunk_scan
 * (bf16 io, the default), or the fused pass described at ssd_fwd_path.
 *
 * chunk_cumsum: reads dt, A; writes G and DT.  One wavefront-level prefix
 *   sum per (b, h, chunk) ("Accelerating Mamba-2 ...", section "Kernel 1").
 * chunk_state: reads x, B, G, DT; writes S.  S_c = X^T diag(w) B with
 *   w_j = dt_j exp2(G_last - G_j) ("Kernel 2", the jump formula with decay).
 * state_passing: reads S, G, init_state; writes h_prev and final_state
 *   ("Kernel 2", the sequential loop over chunks).
 * chunk_scan: reads x, B, C, D, G, DT, h_prev; writes y ("Kernel 3").
 */
ssd_status ssd_chunk_cumsum(const float *dt, const float *A, int64_t chunk_size,
                            const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                            void *stream);
ssd_status ssd_chunk_state(const void *x, const void *B, int64_t chunk_size,
                           const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                           void *stream);
ssd_status ssd_state_passing(const float *init_state, float *final_state, int64_t chunk_size,
                             const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                             void *stream);
ssd_status ssd_chunk_scan(const void *x, const void *B, const void *C, const float *D, void *y,
                          int64_t chunk_size, const ssd_dims *dims, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * chunk_state and state_passing in one sequential pass over the chunks of
 * each (b, h) ("Accelerating Mamba-2 ...", section "Kernel 2": the state is
 * the accumulator of the per-chunk product, stored before each chunk's
 * update).  Reads x, B, G, DT (left by ssd_chunk_cumsum) and init_state
 * (NULL = zeros); writes h_prev and final_state (NULL = not written).  The S
 * region receives B in MFMA fragment order (no chunk state is formed).
 * init_state may equal final_state.  h_prev and final_state agree with those
 * of ssd_chunk_state followed by ssd_state_passing up to fp32 summation
 * order, not bit for bit.
 * bf16 io only: SSD_ERR_UNSUPPORTED for SSD_F32, and for shapes whose
 * per-chunk row span does not fit 32-bit offsets (chunk_size * nheads * 64 * 2
 * or chunk_size * ngroups * dstate * 2 bytes above 2^31 - 1), where
 * ssd_chunked_fwd runs the two stages instead.
 */
ssd_status ssd_state_fwd(const void *x, const void *B, const float *init_state,
                         float *final_state, int64_t chunk_size, const ssd_dims *dims,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The paths of the chunked forward:
 *   SSD_PATH_FOUR_STAGE  chunk_cumsum, chunk_state, state_passing, chunk_scan
 *                        (the per-chunk states S and h_prev go through HBM);
 *   SSD_PATH_STATE_FWD   chunk_cumsum, the one-pass ssd_state_fwd stage
 *                        (h_prev through HBM, S never formed), chunk_scan;
 *   SSD_PATH_FUSED       chunk_cumsum with the per-chunk C B^T tiles, then one
 *                        pass per (b, h) that carries the state through the
 *                        chunks in registers and writes y as it goes (neither
 *                        S nor h_prev exists; x is read once; the chunk-state
 *                        product is taken in fp16, so |B| and |x dt| must stay
 *                        below 65504).  bf16 io; selected only through
 *                        ssd_set_path_override (slower on the shapes measured).
 * All three give y and final_state within the same tolerances; they are
 * not bitwise equal to one another (fp32 summation order).
 */
typedef enum {
    SSD_PATH_FOUR_STAGE = 0,
    SSD_PATH_STATE_FWD = 1,
    SSD_PATH_FUSED = 2
} ssd_fwd_path;

/* The path ssd_chunked_fwd takes for these dims and chunk size (*path, an
 * ssd_fwd_path), under the current override.  Host only; no HIP call. */
ssd_status ssd_chunked_fwd_path(const ssd_dims *dims, int64_t chunk_size, int *path);

/*
 * TEST HOOK, for the parity tests that cover every path: makes later calls
 * in this process take forward path fwd_path (-1 = chosen by the shape; a
 * path the shape does not support is ignored) and, for the one-pass state
 * stage and the backward's one-pass adjoint scan, state_rows / adj_rows sets
 * of 16 state rows per workgroup (4, 2 or 1; 0 = chosen by the shape).  With
 * fwd_path = SSD_PATH_FOUR_STAGE the backward recomputes its states with the
 * four-stage kernels too.  Process-wide and not synchronized with calls on
 * other threads.  (-1, 0, 0) restores the default.  SSD_ERR_UNSUPPORTED for
 * other values.
 */
ssd_status ssd_set_path_override(int32_t fwd_path, int32_t state_rows, int32_t adj_rows);

/*
 * The layer interface around the scan ("Optimizing Nemotron v3 Super in
 * TensorRT-LLM", section 6.1 "The SSU Math" and section 6.3): optional
 * preprocessing of the step and an optional output gate.  Pass NULL for
 * none of them (the plain ssd_chunked_fwd / ssd_decode_step).
 *   dt_bias      float32 [H], added to dt before anything else; NULL = none.
 *   dt_softplus  nonzero: dt <- log(1 + e^dt) where dt <= 20, unchanged
 *                above 20 (after the bias).  Tokens past T stay at dt = 0.
 *   y_io_dtype   0: y (y_t) float32;  1: y (y_t) in the io dtype (bf16 for
 *                bf16 io, rounded to nearest even from the fp32 result; for
 *                fp32 io the same as 0).  Other values SSD_ERR_UNSUPPORTED.
 *   z            gate in x's dtype and layout ([Bt, T, H, P] for the
 *                forward, [Bt, H, P] for decode): y <- y * silu(z) with
 *                silu(z) = z / (1 + e^-z), after the D term.  The state and
 *                final_state are not gated.  NULL = no gate.
 * Pointers are caller-owned device memory, 16-byte aligned (SSD_ERR_ALIGN).
 */
typedef struct {
    const float *dt_bias;
    int32_t dt_softplus;
    int32_t y_io_dtype;
    const void *z;
} ssd_layer_opts;

/* ssd_chunked_fwd with the options above (opts may be NULL). */
ssd_status ssd_chunked_fwd_opts(const void *x, const float *dt, const float *A, const void *B,
                                const void *C, const float *D, int64_t chunk_size,
                                const float *init_state, void *y, float *final_state,
                                const ssd_layer_opts *opts, const ssd_dims *dims,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssd_chunked_fwd_opts without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace is a static device array of
 * SSD_NOALLOC_SCRATCH_BYTES built into the library, one per GPU, held until
 * the process ends.  The call allocates and frees nothing.  The array of the
 * CURRENT device is used (stream must belong to it); its address is looked up
 * on the first call on each device.
 *   - Shapes whose workspace (ssd_chunked_fwd_workspace_size) exceeds
 *     SSD_NOALLOC_SCRATCH_BYTES are rejected with SSD_ERR_WORKSPACE before any
 *     HIP call; nothing is launched or written.  64 MiB holds, e.g., the
 *     370M-layer shape (4 x 2048 tokens, 32 heads, N 128, chunk 256).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (other streams or threads) race and give undefined
 *     results.  Calls in order on one stream are safe; every region a call
 *     reads is written earlier in the same call, so nothing needs clearing
 *     between calls.
 * Other arguments, results and errors as for ssd_chunked_fwd_opts.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ssd_status ssd_chunked_fwd_noalloc(const void *x, const float *dt, const float *A,
                                   const void *B, const void *C, const float *D,
                                   int64_t chunk_size, const float *init_state, void *y,
                                   float *final_state, const ssd_layer_opts *opts,
                                   const ssd_dims *dims, void *stream);

/*
 * One recurrent decode step ("Optimizing Nemotron v3 Super in TensorRT-LLM",
 * section 6.1; "mamba-metal: running Mamba on Apple Silicon", section on
 * O(L) incremental decoding): for every (b, h),
 *     state <- exp(A_h dt_t) state + dt_t x_t (outer) B_t;  y_t = state C_t + D_h x_t
 *
 *   state  [Bt, H, P, N]  float32   in/out, updated in place
 *   x_t    [Bt, H, P]     io dtype  in
 *   dt_t   [Bt, H]        float32   in
 *   B_t, C_t [Bt, G, N]   io dtype  in
 *   A, D   [H]            float32   in
 *   y_t    [Bt, H, P]     float32   out  (io dtype with opts->y_io_dtype)
 * dims->seqlen is ignored.
 */
ssd_status ssd_decode_step(float *state, const void *x_t, const float *dt_t, const void *B_t,
                           const void *C_t, const float *A, const float *D, void *y_t,
                           const ssd_dims *dims, void *stream);

/* ssd_decode_step with the options above (opts may be NULL; z is [Bt, H, P]). */
ssd_status ssd_decode_step_opts(float *state, const void *x_t, const float *dt_t,
                                const void *B_t, const void *C_t, const float *A, const float *D,
                                void *y_t, const ssd_layer_opts *opts, const ssd_dims *dims,
                                void *stream);

/*
 * Several decode steps per sequence in one launch: the multi-token state
 * update of speculative decoding ("Optimizing Nemotron v3 Super in
 * TensorRT-LLM", sections 10.3 and 10.4).  K = dims->seqlen tokens per
 * sequence (0 <= K <= 65536; K = 0 does nothing).  For every (b, h), step
 * k = 0 .. K-1 is the decode step of ssd_decode_step on token k, starting from
 *   - the state passed in, for k = 0;
 *   - the snapshot of step parent[b, k], when parent is given and
 *     0 <= parent[b, k] < k (a draft tree);
 *   - the state after step k - 1, otherwise (any other parent value
 *     included: negative, k itself or a later step).
 *
 *   state      [Bt, H, P, N]     float32   in; out unless NO_STATE_UPDATE
 *   x          [Bt, K, H, P]     io dtype  in
 *   dt         [Bt, K, H]        float32   in
 *   B, C       [Bt, K, G, N]     io dtype  in
 *   A, D       [H]               float32   in
 *   y          [Bt, K, H, P]     float32   out: y of every step (io dtype
 *                                          with opts->y_io_dtype)
 *   snapshots  [Bt, K, H, P, N]  float32   out, or NULL: the state after each
 *                                          step (the buffer a later accept
 *                                          step copies from)
 *   parent     [Bt, K]           int32     in, or NULL (needs snapshots:
 *                                          SSD_ERR_NULL otherwise)
 *   flags      0, or SSD_DECODE_NO_STATE_UPDATE: the state is only read (the
 *              verification pass that must not overwrite the main state);
 *              other bits SSD_ERR_UNSUPPORTED
 *   opts       as for ssd_decode_step_opts, with z [Bt, K, H, P]; may be NULL
 *
 * Without the flag the state ends as the state after step K - 1 (in a tree:
 * that step's own path).  Pointers as for ssd_decode_step (caller-owned device
 * memory, 16-byte aligned, snapshots and parent included); snapshots, y and
 * state must not overlap.  With no tokens (K = 0 or batch 0) the token
 * tensors may be NULL and the state is left as it is.  With K = 1, no parent and no snapshots this is
 * ssd_decode_step(_opts).
 */
#define SSD_DECODE_NO_STATE_UPDATE 1u
ssd_status ssd_decode_multi(float *state, const void *x, const float *dt, const void *B,
                            const void *C, const float *A, const float *D, void *y,
                            float *snapshots, const int32_t *parent, uint32_t flags,
                            const ssd_layer_opts *opts, const ssd_dims *dims, void *stream);

/*
 * The decode state kept at 16 bits per element ("Optimizing Nemotron v3
 * Super in TensorRT-LLM", section 6.5, and the state types of section 6.6):
 *   SSD_STATE_F16    fp16; round to nearest even, or, with philox_rounds in
 *                    1..10, stochastic rounding: |x| + (r / 2^13) ulp16(|x|)
 *                    rounded toward zero and saturated at 65504, r a 13-bit
 *                    field of a word of Philox-4x32 with that many rounds (10
 *                    is the generator's standard; Salmon et al., SC'11): one block
 *                    per 8 consecutive elements of a row, counter = flat index
 *                    (b, h, p, n) of the first (low word, high word, 0, 0),
 *                    key = seed (low word, high word); element n takes word
 *                    (n mod 8) / 2, its bits 0..12 for even n and 16..28 for
 *                    odd n.  Vary the seed from call to call.
 *   SSD_STATE_BF16   bf16, round to nearest even.
 *   SSD_STATE_INT16  int16 codes plus one fp32 decode scale per row (b, h, p)
 *                    in `scale` [Bt, H, P]: the stored value is code * scale;
 *                    after the update, encode = 32767 / max|row| and scale =
 *                    1 / encode (fp32 divisions), code = round-half-even(x *
 *                    encode); an all-zero row stores codes 0 and scale 0.
 *   SSD_STATE_F32    the fp32 state of ssd_decode_step.
 * philox_rounds must be 0 except for SSD_STATE_F16; scale is required for
 * SSD_STATE_INT16 and must be NULL otherwise (SSD_ERR_UNSUPPORTED / _NULL).
 */
typedef enum {
    SSD_STATE_F32 = 0,
    SSD_STATE_F16 = 1,
    SSD_STATE_BF16 = 2,
    SSD_STATE_INT16 = 3
} ssd_state_dtype;

typedef struct {
    int32_t dtype;        /* ssd_state_dtype */
    int32_t philox_rounds; /* SSD_STATE_F16 only: 0 = nearest, 1..10 = stochastic */
    uint64_t seed;        /* Philox key for stochastic rounding */
    float *scale;         /* SSD_STATE_INT16: [Bt, H, P] decode scales, in/out */
} ssd_state_format;

/*
 * ssd_decode_step on a state stored as *fmt says: the stored state is decoded
 * to fp32, updated and y computed exactly as in ssd_decode_step (y from the
 * updated fp32 state), and the new state stored back in the same format, in
 * place.  state is [Bt, H, P, N] of 16-bit elements (fp32 for
 * SSD_STATE_F32).  Other arguments, options and errors as for
 * ssd_decode_step_opts.
 */
ssd_status ssd_decode_step_lp(void *state, const ssd_state_format *fmt, const void *x_t,
                              const float *dt_t, const void *B_t, const void *C_t, const float *A,
                              const float *D, void *y_t, const ssd_layer_opts *opts,
                              const ssd_dims *dims, void *stream);

/*
 * The backward of ssd_chunked_fwd (no layer options): gradients of
 * L = sum(dy . y) + sum(dfinal . final_state).  The "mamba3" kernel card,
 * section "Backward": the forward's chunk states are recomputed on the
 * workspace, the state adjoint is scanned in reverse over the chunks between
 * two chunk-parallel passes, and there are no floating-point atomics: every
 * output element has one owner and every sum over heads or batch rows is
 * taken in a fixed order, so reruns are bitwise identical.  Gradients are
 * float32 whatever the io dtype.
 *
 *   x, dt, A, B, C, D, chunk_size, init_state, dims   as for ssd_chunked_fwd
 *   dy      [Bt, T, H, P]   float32  in   gradient of y
 *   dfinal  [Bt, H, P, N]   float32  in   gradient of the final state, or NULL (0)
 *   dx      [Bt, T, H, P]   float32  out
 *   ddt     [Bt, T, H]      float32  out
 *   dA, dD  [H]             float32  out  (summed over batch and tokens)
 *   dB, dC  [Bt, T, G, N]   float32  out  (summed over the heads of a group)
 *   dinit   [Bt, H, P, N]   float32  out  gradient of init_state, or NULL (not
 *                                         written); defined for init_state = NULL too
 * workspace: ssd_chunked_bwd_workspace_size(dims, chunk_size) bytes, 16-byte
 * aligned.  With no tokens the token tensors may be NULL; dA and dD are then
 * zero and dinit = dfinal.  Errors as for ssd_chunked_fwd.
 */
size_t ssd_chunked_bwd_workspace_size(const ssd_dims *dims, int64_t chunk_size);
ssd_status ssd_chunked_bwd(const void *x, const float *dt, const float *A, const void *B,
                           const void *C, const float *D, int64_t chunk_size,
                           const float *init_state, const float *dy, const float *dfinal,
                           float *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                           float *dinit, const ssd_dims *dims, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Static text for a status code. */
const char *ssd_status_string(ssd_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *ssd_last_error_detail(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
