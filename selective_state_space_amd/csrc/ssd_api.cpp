// C ABI of libssd.so: host-side validation, workspace layout, and the launch
// sequence of the chunked forward (chunk_cumsum -> chunk_state ->
// state_passing -> chunk_scan, "Accelerating Mamba-2 with High-Performance
// Forward Pass Kernels in NVIDIA CUDA Tile", sections "Kernel 1" to "Kernel
// 3"; for bf16 io and enough (batch, head) chains the middle two run as one
// pass, as in that page's "Kernel 2") and of the decode step ("Optimizing Nemotron v3 Super in
// TensorRT-LLM", section 6.1).
//
// Every check runs on the host before the first HIP call, so a rejected call
// launches and writes nothing; the "mamba3" kernel card ("Requirements and
// limits") likewise checks its requirements up front and names the figures.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/ssd.h"
#include "ssd_launch.h"

// The workspace of ssd_chunked_fwd_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes its
// name to a kernel (on the host the name is only a stand-in): the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_detail[512] = "";

ssd_status fail(ssd_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return st;
}

ssd_status ok() {
    g_detail[0] = '\0';
    return SSD_OK;
}

bool debug_sync() {
    static const int on = [] {
        const char *e = getenv("SSD_DEBUG_SYNC");
        return (e && e[0] && e[0] != '0') ? 1 : 0;
    }();
    return on != 0;
}

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr uint64_t kMaxGrid = (uint64_t(1) << 31) - 1;
constexpr int64_t kMaxTokensPerStep = int64_t(1) << 16;   // ssd_decode_multi's K

bool misaligned(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Validates dims (and chunk_size when L > 0) and fills `s`.
ssd_status check_dims(const ssd_dims *d, int64_t L, bool need_seq, ssd::Shape *s) {
    if (!d) return fail(SSD_ERR_NULL, "dims is NULL");
    if (d->batch < 0 || d->batch > kMaxDim)
        return fail(SSD_ERR_SHAPE, "batch = %lld out of range [0, 2^30]", (long long)d->batch);
    if (need_seq && (d->seqlen < 0 || d->seqlen > (int64_t(1) << 40)))
        return fail(SSD_ERR_SHAPE, "seqlen = %lld out of range [0, 2^40]", (long long)d->seqlen);
    if (d->nheads < 1 || d->nheads > kMaxDim)
        return fail(SSD_ERR_SHAPE, "nheads = %lld must be >= 1", (long long)d->nheads);
    if (d->ngroups < 1 || d->ngroups > d->nheads)
        return fail(SSD_ERR_SHAPE, "ngroups = %lld must be in [1, nheads = %lld]",
                    (long long)d->ngroups, (long long)d->nheads);
    if (d->nheads % d->ngroups)
        return fail(SSD_ERR_SHAPE, "nheads = %lld is not a multiple of ngroups = %lld",
                    (long long)d->nheads, (long long)d->ngroups);
    if (d->headdim < 1 || d->dstate < 1)
        return fail(SSD_ERR_SHAPE, "headdim = %lld and dstate = %lld must be >= 1",
                    (long long)d->headdim, (long long)d->dstate);
    if (d->headdim != 64)
        return fail(SSD_ERR_UNSUPPORTED, "headdim = %lld; only 64 is instantiated",
                    (long long)d->headdim);
    if (d->dstate != 64 && d->dstate != 128)
        return fail(SSD_ERR_UNSUPPORTED, "dstate = %lld; only 64 and 128 are instantiated",
                    (long long)d->dstate);
    if (d->io_dtype != SSD_F32 && d->io_dtype != SSD_BF16)
        return fail(SSD_ERR_UNSUPPORTED, "io_dtype = %d; only SSD_F32 (0) and SSD_BF16 (1)",
                    (int)d->io_dtype);
    if (L > 0 || need_seq) {
        if (L != 64 && L != 128 && L != 256)
            return fail(SSD_ERR_UNSUPPORTED, "chunk_size = %lld; only 64, 128, 256 are instantiated",
                        (long long)L);
    }
    s->Bt = d->batch;
    s->T = need_seq ? d->seqlen : 1;
    s->H = d->nheads;
    s->P = d->headdim;
    s->N = d->dstate;
    s->G = d->ngroups;
    s->L = L > 0 ? L : 64;
    s->nc = need_seq ? (s->T + s->L - 1) / s->L : 0;
    s->bf16 = d->io_dtype == SSD_BF16;
    s->ybf16 = false;
    if (s->nc > kMaxDim) return fail(SSD_ERR_SHAPE, "too many chunks (%lld)", (long long)s->nc);
    const uint64_t grid_chunks = (uint64_t)s->Bt * (uint64_t)s->nc * (uint64_t)s->H;
    const uint64_t grid_heads = (uint64_t)s->Bt * (uint64_t)s->H * 8u;
    if (grid_chunks > kMaxGrid || grid_heads > kMaxGrid)
        return fail(SSD_ERR_SHAPE, "problem too large for one launch (batch*chunks*heads = %llu)",
                    (unsigned long long)grid_chunks);
    return SSD_OK;
}

struct Layout {
    size_t off[4];
    size_t total;
};

Layout layout_of(const ssd::Shape &s) {
    Layout l;
    const size_t units = (size_t)s.Bt * s.H * s.nc;
    const size_t g = units * s.L * sizeof(float);
    // S, or on the one-pass state path B in MFMA fragment order
    size_t st = units * s.P * s.N * sizeof(float);
    if (ssd::state_fwd_bfrag_bytes(s) > st) st = ssd::state_fwd_bfrag_bytes(s);
    // h_prev, or on the fused path the C B^T tiles
    size_t hp = units * s.P * s.N * (s.bf16 ? 2 : 4);
    if (s.bf16 && ssd::fused_cbt_bytes(s) > hp) hp = ssd::fused_cbt_bytes(s);
    l.off[0] = 0;
    l.off[1] = align256(l.off[0] + g);
    l.off[2] = align256(l.off[1] + g);
    l.off[3] = align256(l.off[2] + st);
    l.total = units ? align256(l.off[3] + hp) : 0;
    return l;
}

struct Ws {
    float *G, *DT, *S;
    void *hprev;
};

ssd_status check_ws(const ssd::Shape &s, void *ws, size_t bytes, Ws *w) {
    const Layout l = layout_of(s);
    if (l.total && !ws) return fail(SSD_ERR_NULL, "workspace is NULL (%zu bytes needed)", l.total);
    if (misaligned(ws)) return fail(SSD_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (bytes < l.total)
        return fail(SSD_ERR_WORKSPACE, "workspace_bytes = %zu < %zu required", bytes, l.total);
    char *base = static_cast<char *>(ws);
    w->G = reinterpret_cast<float *>(base + l.off[0]);
    w->DT = reinterpret_cast<float *>(base + l.off[1]);
    w->S = reinterpret_cast<float *>(base + l.off[2]);
    w->hprev = base + l.off[3];
    return SSD_OK;
}

#define REQUIRE_PTR(p)                                                          \
    do {                                                                        \
        if (!(p)) return fail(SSD_ERR_NULL, "%s is NULL", #p);                  \
        if (misaligned(p)) return fail(SSD_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
    } while (0)
#define OPTIONAL_PTR(p)                                                         \
    do {                                                                        \
        if (misaligned(p)) return fail(SSD_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
    } while (0)

// The optional layer interface: pointers 16-byte aligned.  Also records in
// the shape whether y is stored in the io dtype (bf16 io only: for fp32 io
// the io dtype is float32 already).
ssd_status check_opts(const ssd_layer_opts *o, ssd::Shape *s) {
    if (!o) return SSD_OK;
    if (o->y_io_dtype != 0 && o->y_io_dtype != 1)
        return fail(SSD_ERR_UNSUPPORTED, "ssd_layer_opts.y_io_dtype = %d; 0 or 1",
                    (int)o->y_io_dtype);
    if (misaligned(o->dt_bias)) return fail(SSD_ERR_ALIGN, "dt_bias is not 16-byte aligned");
    if (misaligned(o->z)) return fail(SSD_ERR_ALIGN, "z is not 16-byte aligned");
    s->ybf16 = s->bf16 && o->y_io_dtype != 0;
    return SSD_OK;
}

ssd_status hip_result(hipError_t e, const char *what, hipStream_t st) {
    if (e == hipSuccess && debug_sync()) {
        e = hipStreamSynchronize(st);
        if (e == hipSuccess) e = hipGetLastError();
    }
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return SSD_OK;
}

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; later calls read it without a
// lock.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

ssd_status scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SSD_ERR_UNSUPPORTED, "device %d: the scratch table holds %d devices", dev,
                    kMaxDevices);
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return fail(SSD_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(e));
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SSD_OK;
}

// Stage runners on validated arguments.
// B non-NULL: also lay B out for the one-pass state stage (bf16 only), in
// bfrag (default: w.S).
ssd_status run_cumsum(const ssd::Shape &s, const float *dt, const float *A, const Ws &w,
                      hipStream_t st, const ssd_layer_opts *o = nullptr,
                      const void *B = nullptr, void *bfrag = nullptr) {
    if (B && !bfrag) bfrag = w.S;
    return hip_result(ssd::launch_chunk_cumsum(s, dt, A, w.G, w.DT, o ? o->dt_bias : nullptr,
                                               o ? o->dt_softplus : 0, st, B,
                                               B ? bfrag : nullptr),
                      "chunk_cumsum", st);
}
ssd_status run_state(const ssd::Shape &s, const void *x, const void *B, const Ws &w,
                     hipStream_t st) {
    return hip_result(ssd::launch_chunk_state(s, x, B, w.G, w.DT, w.S, st), "chunk_state", st);
}
ssd_status run_passing(const ssd::Shape &s, const float *init, float *fin, const Ws &w,
                       hipStream_t st) {
    return hip_result(ssd::launch_state_passing(s, w.S, w.G, init, w.hprev, fin, st),
                      "state_passing", st);
}
// Path override for tests (ssd_set_path_override): -1 / 0 = chosen by the
// shape.  Set between calls, read by every call; never from the environment.
struct PathOverride {
    int fwd_path = -1;     // an ssd_fwd_path, or -1
    int state_rows = 0;    // 4, 2, 1, or 0
    int adj_rows = 0;      // 4, 2, 1, or 0
};
PathOverride g_override;

int state_fwd_rows() { return g_override.state_rows; }
int state_adj_rows() { return g_override.adj_rows; }

// The forward path a call takes: the override where the shape supports it,
// else the shape's own choice: the one-pass state stage for bf16 io (measured
// fastest at the 370M, 2.7B and long-context shapes, ahead of the four stages
// and of the fused pass), the four stages for fp32 io.
int fwd_path(const ssd::Shape &s) {
    const bool one_pass_ok = ssd::state_fwd_supported(s);
    const bool fused_ok = ssd::fused_fwd_supported(s);
    switch (g_override.fwd_path) {
    case SSD_PATH_FOUR_STAGE: return SSD_PATH_FOUR_STAGE;
    case SSD_PATH_STATE_FWD:
        if (one_pass_ok) return SSD_PATH_STATE_FWD;
        break;
    case SSD_PATH_FUSED:
        if (fused_ok) return SSD_PATH_FUSED;
        break;
    default: break;
    }
    if (one_pass_ok && ssd::state_fwd_preferred(s)) return SSD_PATH_STATE_FWD;
    return SSD_PATH_FOUR_STAGE;
}
bool use_state_fwd(const ssd::Shape &s) { return fwd_path(s) == SSD_PATH_STATE_FWD; }
// The backward recomputes the forward's states with the one-pass stage
// wherever it is supported, unless the override asks for the four stages.
bool bwd_one_pass(const ssd::Shape &s) {
    return ssd::state_fwd_supported(s) && g_override.fwd_path != SSD_PATH_FOUR_STAGE;
}
// bfrag_ready: run_cumsum was given B, so w.S already holds its fragments.
ssd_status run_state_fwd(const ssd::Shape &s, const void *x, const void *B, const float *init,
                         float *fin, const Ws &w, hipStream_t st, bool bfrag_ready = false) {
    return hip_result(ssd::launch_state_fwd(s, x, B, w.G, w.DT, init, w.hprev, fin, w.S,
                                            state_fwd_rows(), false, st, bfrag_ready),
                      "state_fwd", st);
}
ssd_status run_scan(const ssd::Shape &s, const void *x, const void *B, const void *C,
                    const float *D, void *y, const Ws &w, hipStream_t st,
                    const void *z = nullptr) {
    return hip_result(ssd::launch_chunk_scan(s, x, B, C, D, w.G, w.DT, w.hprev, y, z, st),
                      "chunk_scan", st);
}

}  // namespace

extern "C" {

size_t ssd_chunked_fwd_workspace_size(const ssd_dims *dims, int64_t chunk_size) {
    ssd::Shape s;
    if (check_dims(dims, chunk_size, true, &s) != SSD_OK) return 0;
    return layout_of(s).total;
}

ssd_status ssd_chunked_fwd_workspace_layout(const ssd_dims *dims, int64_t chunk_size,
                                            size_t offsets[4]) {
    if (!offsets) return fail(SSD_ERR_NULL, "offsets is NULL");
    ssd::Shape s;
    const ssd_status r = check_dims(dims, chunk_size, true, &s);
    if (r != SSD_OK) return r;
    const Layout l = layout_of(s);
    for (int i = 0; i < 4; ++i) offsets[i] = l.off[i];
    return ok();
}

ssd_status ssd_chunk_cumsum(const float *dt, const float *A, int64_t chunk_size,
                            const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                            void *stream) {
    ssd::Shape s;
    ssd_status r = check_dims(dims, chunk_size, true, &s);
    if (r != SSD_OK) return r;
    REQUIRE_PTR(dt);
    REQUIRE_PTR(A);
    Ws w;
    if ((r = check_ws(s, workspace, workspace_bytes, &w)) != SSD_OK) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((r = run_cumsum(s, dt, A, w, st)) != SSD_OK) return r;
    return ok();
}

ssd_status ssd_chunk_state(const void *x, const void *B, int64_t chunk_size, const ssd_dims *dims,
                           void *workspace, size_t workspace_bytes, void *stream) {
    ssd::Shape s;
    ssd_status r = check_dims(dims, chunk_size, true, &s);
    if (r != SSD_OK) return r;
    REQUIRE_PTR(x);
    REQUIRE_PTR(B);
    Ws w;
    if ((r = check_ws(s, workspace, workspace_bytes, &w)) != SSD_OK) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((r = run_state(s, x, B, w, st)) != SSD_OK) return r;
    return ok();
}

ssd_status ssd_state_passing(const float *init_state, float *final_state, int64_t chunk_size,
                             const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                             void *stream) {
    ssd::Shape s;
    ssd_status r = check_dims(dims, chunk_size, true, &s);
    if (r != SSD_OK) return r;
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(final_state);
    Ws w;
    if ((r = check_ws(s, workspace, workspace_bytes, &w)) != SSD_OK) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((r = run_passing(s, init_state, final_state, w, st)) != SSD_OK) return r;
    return ok();
}

ssd_status ssd_chunk_scan(const void *x, const void *B, const void *C, const float *D, void *y,
                          int64_t chunk_size, const ssd_dims *dims, void *workspace,
                          size_t workspace_bytes, void *stream) {
    ssd::Shape s;
    ssd_status r = check_dims(dims, chunk_size, true, &s);
    if (r != SSD_OK) return r;
    REQUIRE_PTR(x);
    REQUIRE_PTR(B);
    REQUIRE_PTR(C);
    REQUIRE_PTR(D);
    REQUIRE_PTR(y);
    Ws w;
    if ((r = check_ws(s, workspace, workspace_bytes, &w)) != SSD_OK) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((r = run_scan(s, x, B, C, D, y, w, st)) != SSD_OK) return r;
    return ok();
}

ssd_status ssd_state_fwd(const void *x, const void *B, const float *init_state,
                         float *final_state, int64_t chunk_size, const ssd_dims *dims,
                         void *workspace, size_t workspace_bytes, void *stream) {
    ssd::Shape s;
    ssd_status r = check_dims(dims, chunk_size, true, &s);
    if (r != SSD_OK) return r;
    if (!ssd::state_fwd_supported(s))
        return fail(SSD_ERR_UNSUPPORTED,
                    "ssd_state_fwd needs bf16 io and per-chunk row spans below 2^31 bytes");
    if (s.Bt > 0 && s.T > 0) {
        REQUIRE_PTR(x);
        REQUIRE_PTR(B);
    } else {
        OPTIONAL_PTR(x);
        OPTIONAL_PTR(B);
    }
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(final_state);
    Ws w;
    if ((r = check_ws(s, workspace, workspace_bytes, &w)) != SSD_OK) return r;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((r = run_state_fwd(s, x, B, init_state, final_state, w, st)) != SSD_OK) return r;
    return ok();
}

ssd_status ssd_chunked_fwd_path(const ssd_dims *dims, int64_t chunk_size, int *path) {
    if (!path) return fail(SSD_ERR_NULL, "path is NULL");
    ssd::Shape s;
    const ssd_status r = check_dims(dims, chunk_size, true, &s);
    if (r != SSD_OK) return r;
    *path = fwd_path(s);
    return ok();
}

ssd_status ssd_set_path_override(int32_t fwd, int32_t state_rows, int32_t adj_rows) {
    if (fwd < -1 || fwd > SSD_PATH_FUSED)
        return fail(SSD_ERR_UNSUPPORTED, "fwd_path = %d; -1 or an ssd_fwd_path", (int)fwd);
    auto rows_ok = [](int32_t r) { return r == 0 || r == 1 || r == 2 || r == 4; };
    if (!rows_ok(state_rows))
        return fail(SSD_ERR_UNSUPPORTED, "state_rows = %d; 0, 1, 2 or 4", (int)state_rows);
    if (!rows_ok(adj_rows))
        return fail(SSD_ERR_UNSUPPORTED, "adj_rows = %d; 0, 1, 2 or 4", (int)adj_rows);
    g_override.fwd_path = fwd;
    g_override.state_rows = state_rows;
    g_override.adj_rows = adj_rows;
    return ok();
}

ssd_status ssd_chunked_fwd_opts(const void *x, const float *dt, const float *A, const void *B,
                                const void *C, const float *D, int64_t chunk_size,
                                const float *init_state, void *y, float *final_state,
                                const ssd_layer_opts *opts, const ssd_dims *dims,
                                void *workspace, size_t workspace_bytes, void *stream) {
    ssd::Shape s;
    ssd_status r = check_dims(dims, chunk_size, true, &s);
    if (r != SSD_OK) return r;
    if ((r = check_opts(opts, &s)) != SSD_OK) return r;
    if (s.Bt > 0 && s.T > 0) {
        REQUIRE_PTR(x);
        REQUIRE_PTR(dt);
        REQUIRE_PTR(A);
        REQUIRE_PTR(B);
        REQUIRE_PTR(C);
        REQUIRE_PTR(D);
        REQUIRE_PTR(y);
    } else {  // no tokens: the token tensors are empty and may be NULL
        OPTIONAL_PTR(x);
        OPTIONAL_PTR(dt);
        OPTIONAL_PTR(A);
        OPTIONAL_PTR(B);
        OPTIONAL_PTR(C);
        OPTIONAL_PTR(D);
        OPTIONAL_PTR(y);
    }
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(final_state);
    Ws w;
    if ((r = check_ws(s, workspace, workspace_bytes, &w)) != SSD_OK) return r;
    if (s.Bt == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int path = fwd_path(s);
    if (path == SSD_PATH_FUSED) {
        // the cumsum, B fragments and C B^T tiles in one launch, then the pass
        r = hip_result(ssd::launch_fused_prep(s, dt, A, w.G, w.DT, opts ? opts->dt_bias : nullptr,
                                              opts ? opts->dt_softplus : 0, B, C, w.S, w.hprev,
                                              st),
                       "fused_prep", st);
        if (r != SSD_OK) return r;
        r = hip_result(ssd::launch_fused_fwd(s, x, C, D, w.G, w.DT, w.S, w.hprev, init_state,
                                             final_state, y, opts ? opts->z : nullptr, st),
                       "fused_fwd", st);
        if (r != SSD_OK) return r;
        return ok();
    }
    const bool one_pass = path == SSD_PATH_STATE_FWD;
    // the one-pass state stage's B fragments are built in the cumsum's launch
    if ((r = run_cumsum(s, dt, A, w, st, opts, one_pass ? B : nullptr)) != SSD_OK) return r;
    if (one_pass) {
        if ((r = run_state_fwd(s, x, B, init_state, final_state, w, st, true)) != SSD_OK)
            return r;
    } else {
        if ((r = run_state(s, x, B, w, st)) != SSD_OK) return r;
        if ((r = run_passing(s, init_state, final_state, w, st)) != SSD_OK) return r;
    }
    if ((r = run_scan(s, x, B, C, D, y, w, st, opts ? opts->z : nullptr)) != SSD_OK) return r;
    return ok();
}

ssd_status ssd_chunked_fwd(const void *x, const float *dt, const float *A, const void *B,
                           const void *C, const float *D, int64_t chunk_size,
                           const float *init_state, void *y, float *final_state,
                           const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                           void *stream) {
    return ssd_chunked_fwd_opts(x, dt, A, B, C, D, chunk_size, init_state, y, final_state,
                                nullptr, dims, workspace, workspace_bytes, stream);
}

ssd_status ssd_chunked_fwd_noalloc(const void *x, const float *dt, const float *A,
                                   const void *B, const void *C, const float *D,
                                   int64_t chunk_size, const float *init_state, void *y,
                                   float *final_state, const ssd_layer_opts *opts,
                                   const ssd_dims *dims, void *stream) {
    ssd::Shape s;
    ssd_status r = check_dims(dims, chunk_size, true, &s);
    if (r != SSD_OK) return r;
    // the size check is host arithmetic only: a shape that does not fit is
    // rejected before any HIP call
    const size_t need = layout_of(s).total;
    if (need > (size_t)SSD_NOALLOC_SCRATCH_BYTES)
        return fail(SSD_ERR_WORKSPACE,
                    "this shape needs %zu bytes of workspace; the static scratch of "
                    "ssd_chunked_fwd_noalloc holds %zu",
                    need, (size_t)SSD_NOALLOC_SCRATCH_BYTES);
    if (s.Bt == 0 || need == 0)   // nothing to compute (the usual checks still apply)
        return ssd_chunked_fwd_opts(x, dt, A, B, C, D, chunk_size, init_state, y, final_state,
                                    opts, dims, nullptr, 0, stream);
    void *ws = nullptr;
    if ((r = scratch_of_current_device(&ws)) != SSD_OK) return r;
    return ssd_chunked_fwd_opts(x, dt, A, B, C, D, chunk_size, init_state, y, final_state, opts,
                                dims, ws, (size_t)SSD_NOALLOC_SCRATCH_BYTES, stream);
}

ssd_status ssd_decode_step_opts(float *state, const void *x_t, const float *dt_t,
                                const void *B_t, const void *C_t, const float *A, const float *D,
                                void *y_t, const ssd_layer_opts *opts, const ssd_dims *dims,
                                void *stream) {
    ssd::Shape s;
    ssd_status r = check_dims(dims, 0, false, &s);
    if (r != SSD_OK) return r;
    if ((r = check_opts(opts, &s)) != SSD_OK) return r;
    REQUIRE_PTR(state);
    REQUIRE_PTR(x_t);
    REQUIRE_PTR(dt_t);
    REQUIRE_PTR(B_t);
    REQUIRE_PTR(C_t);
    REQUIRE_PTR(A);
    REQUIRE_PTR(D);
    REQUIRE_PTR(y_t);
    if (s.Bt == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    r = hip_result(ssd::launch_decode_step(s, state, x_t, dt_t, B_t, C_t, A, D, y_t,
                                           opts ? opts->dt_bias : nullptr,
                                           opts ? opts->dt_softplus : 0, opts ? opts->z : nullptr,
                                           st),
                   "decode_step", st);
    if (r != SSD_OK) return r;
    return ok();
}

ssd_status ssd_decode_step(float *state, const void *x_t, const float *dt_t, const void *B_t,
                           const void *C_t, const float *A, const float *D, void *y_t,
                           const ssd_dims *dims, void *stream) {
    return ssd_decode_step_opts(state, x_t, dt_t, B_t, C_t, A, D, y_t, nullptr, dims, stream);
}

ssd_status ssd_decode_multi(float *state, const void *x, const float *dt, const void *B,
                            const void *C, const float *A, const float *D, void *y,
                            float *snapshots, const int32_t *parent, uint32_t flags,
                            const ssd_layer_opts *opts, const ssd_dims *dims, void *stream) {
    ssd::Shape s;
    ssd_status r = check_dims(dims, 0, false, &s);
    if (r != SSD_OK) return r;
    if (dims->seqlen < 0 || dims->seqlen > kMaxTokensPerStep)
        return fail(SSD_ERR_SHAPE, "seqlen = %lld tokens per sequence out of range [0, %lld]",
                    (long long)dims->seqlen, (long long)kMaxTokensPerStep);
    s.T = dims->seqlen;
    if ((double)s.Bt * (double)s.T * (double)s.H * 64.0 * (double)s.N * 4.0 > 0x1p50)
        return fail(SSD_ERR_SHAPE, "batch * seqlen * nheads too large for 64-bit offsets");
    if (flags & ~(uint32_t)SSD_DECODE_NO_STATE_UPDATE)
        return fail(SSD_ERR_UNSUPPORTED, "flags = 0x%x; only SSD_DECODE_NO_STATE_UPDATE is defined",
                    (unsigned)flags);
    if ((r = check_opts(opts, &s)) != SSD_OK) return r;
    if (s.Bt > 0)
        REQUIRE_PTR(state);
    else
        OPTIONAL_PTR(state);
    if (s.Bt > 0 && s.T > 0) {
        REQUIRE_PTR(x);
        REQUIRE_PTR(dt);
        REQUIRE_PTR(B);
        REQUIRE_PTR(C);
        REQUIRE_PTR(A);
        REQUIRE_PTR(D);
        REQUIRE_PTR(y);
    } else {  // no tokens: the token tensors are empty and may be NULL
        OPTIONAL_PTR(x);
        OPTIONAL_PTR(dt);
        OPTIONAL_PTR(B);
        OPTIONAL_PTR(C);
        OPTIONAL_PTR(A);
        OPTIONAL_PTR(D);
        OPTIONAL_PTR(y);
    }
    if (misaligned(snapshots)) return fail(SSD_ERR_ALIGN, "snapshots is not 16-byte aligned");
    if (misaligned(parent)) return fail(SSD_ERR_ALIGN, "parent is not 16-byte aligned");
    if (parent && !snapshots)
        return fail(SSD_ERR_NULL, "parent needs the snapshots buffer (steps restart from it)");
    if (s.Bt == 0 || s.T == 0) return ok();
    ssd::MultiArgs m{state, x, dt, B, C, A, D, static_cast<float *>(y),
                     opts ? opts->dt_bias : nullptr, opts ? opts->dt_softplus : 0,
                     opts ? opts->z : nullptr, snapshots, parent,
                     (flags & SSD_DECODE_NO_STATE_UPDATE) ? 0 : 1};
    hipStream_t st = static_cast<hipStream_t>(stream);
    r = hip_result(ssd::launch_decode_multi(s, m, st), "decode_multi", st);
    if (r != SSD_OK) return r;
    return ok();
}

ssd_status ssd_decode_step_lp(void *state, const ssd_state_format *fmt, const void *x_t,
                              const float *dt_t, const void *B_t, const void *C_t, const float *A,
                              const float *D, void *y_t, const ssd_layer_opts *opts,
                              const ssd_dims *dims, void *stream) {
    if (!fmt) return fail(SSD_ERR_NULL, "fmt is NULL");
    const int32_t f = fmt->dtype;
    if (f != SSD_STATE_F32 && f != SSD_STATE_F16 && f != SSD_STATE_BF16 && f != SSD_STATE_INT16)
        return fail(SSD_ERR_UNSUPPORTED, "state dtype = %d; only SSD_STATE_F32/F16/BF16/INT16",
                    (int)f);
    if (fmt->philox_rounds != 0 &&
        (fmt->philox_rounds < 1 || fmt->philox_rounds > 10 || f != SSD_STATE_F16))
        return fail(SSD_ERR_UNSUPPORTED,
                    "philox_rounds = %d; 1..10 (stochastic rounding) for SSD_STATE_F16 only",
                    (int)fmt->philox_rounds);
    if (f == SSD_STATE_INT16 && !fmt->scale)
        return fail(SSD_ERR_NULL, "fmt->scale is NULL (SSD_STATE_INT16 needs its row scales)");
    if (f != SSD_STATE_INT16 && fmt->scale)
        return fail(SSD_ERR_UNSUPPORTED, "fmt->scale is only used by SSD_STATE_INT16");
    if (misaligned(fmt->scale)) return fail(SSD_ERR_ALIGN, "fmt->scale is not 16-byte aligned");
    if (f == SSD_STATE_F32)
        return ssd_decode_step_opts(static_cast<float *>(state), x_t, dt_t, B_t, C_t, A, D, y_t,
                                    opts, dims, stream);
    ssd::Shape s;
    ssd_status r = check_dims(dims, 0, false, &s);
    if (r != SSD_OK) return r;
    if ((r = check_opts(opts, &s)) != SSD_OK) return r;
    REQUIRE_PTR(state);
    REQUIRE_PTR(x_t);
    REQUIRE_PTR(dt_t);
    REQUIRE_PTR(B_t);
    REQUIRE_PTR(C_t);
    REQUIRE_PTR(A);
    REQUIRE_PTR(D);
    REQUIRE_PTR(y_t);
    if (s.Bt == 0) return ok();
    const int lf = f == SSD_STATE_F16 ? ssd::LOWP_F16
                                      : (f == SSD_STATE_BF16 ? ssd::LOWP_BF16 : ssd::LOWP_INT16);
    ssd::LowpArgs a{state, fmt->scale, lf, (int)fmt->philox_rounds, fmt->seed, x_t, dt_t, B_t, C_t,
                    A, D, static_cast<float *>(y_t), opts ? opts->dt_bias : nullptr,
                    opts ? opts->dt_softplus : 0, opts ? opts->z : nullptr};
    hipStream_t st = static_cast<hipStream_t>(stream);
    r = hip_result(ssd::launch_decode_lowp(s, a, st), "decode_lowp", st);
    if (r != SSD_OK) return r;
    return ok();
}

// Backward workspace: the forward's regions, then the final state, C B^T per
// (b, chunk, group) (fp32 for fp32 io; for bf16 io it and its transpose as
// three bf16 terms each, the dB/dC matrix M and the C fragments of the
// adjoint scan), three planes of per-token scalars, 3 * Bt*H fp64 partials and,
// for bf16 io, h_prev again in fp32 (the forward keeps it in bf16 for its
// MFMA; the decay gradient sums per-token products of it over the whole
// sequence, where bf16's rounding would not cancel).
struct BwdLayout {
    Layout fwd;
    size_t fin, cb, cb3, cbt3, mt, cfr, tok, part, hp32, total;
};

BwdLayout bwd_layout_of(const ssd::Shape &s) {
    BwdLayout l;
    l.fwd = layout_of(s);
    const size_t bh = (size_t)s.Bt * s.H;
    l.fin = align256(l.fwd.total);
    l.cb = align256(l.fin + bh * s.P * s.N * sizeof(float));
    l.cb3 = align256(l.cb + (s.bf16 ? 0 : ssd::bwd_cb_bytes(s)));
    l.cbt3 = align256(l.cb3 + (s.bf16 ? ssd::bwd_cb_bytes(s) * 3 / 2 : 0));
    l.mt = align256(l.cbt3 + (s.bf16 ? ssd::bwd_cb_bytes(s) * 3 / 2 : 0));
    l.cfr = align256(l.mt + (s.bf16 ? ssd::bwd_cb_bytes(s) : 0));
    l.tok = align256(l.cfr + (ssd::state_adj_supported(s) ? ssd::state_fwd_bfrag_bytes(s) : 0));
    l.part = align256(l.tok + 3 * bh * s.nc * s.L * sizeof(float));
    l.hp32 = align256(l.part + 3 * bh * sizeof(double));
    const size_t hp = s.bf16 ? bh * s.nc * s.P * s.N * sizeof(float) : 0;
    l.total = bh ? align256(l.hp32 + hp) : 0;
    return l;
}

size_t ssd_chunked_bwd_workspace_size(const ssd_dims *dims, int64_t chunk_size) {
    ssd::Shape s;
    if (check_dims(dims, chunk_size, true, &s) != SSD_OK) return 0;
    return bwd_layout_of(s).total;
}

ssd_status ssd_chunked_bwd(const void *x, const float *dt, const float *A, const void *B,
                           const void *C, const float *D, int64_t chunk_size,
                           const float *init_state, const float *dy, const float *dfinal,
                           float *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                           float *dinit, const ssd_dims *dims, void *workspace,
                           size_t workspace_bytes, void *stream) {
    ssd::Shape s;
    ssd_status r = check_dims(dims, chunk_size, true, &s);
    if (r != SSD_OK) return r;
    if (s.Bt > 0 && s.T > 0) {
        REQUIRE_PTR(x);
        REQUIRE_PTR(dt);
        REQUIRE_PTR(B);
        REQUIRE_PTR(C);
        REQUIRE_PTR(dy);
        REQUIRE_PTR(dx);
        REQUIRE_PTR(ddt);
        REQUIRE_PTR(dB);
        REQUIRE_PTR(dC);
    } else {  // no tokens: the token tensors are empty and may be NULL
        OPTIONAL_PTR(x);
        OPTIONAL_PTR(dt);
        OPTIONAL_PTR(B);
        OPTIONAL_PTR(C);
        OPTIONAL_PTR(dy);
        OPTIONAL_PTR(dx);
        OPTIONAL_PTR(ddt);
        OPTIONAL_PTR(dB);
        OPTIONAL_PTR(dC);
    }
    REQUIRE_PTR(A);
    REQUIRE_PTR(D);
    REQUIRE_PTR(dA);
    REQUIRE_PTR(dD);
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(dfinal);
    OPTIONAL_PTR(dinit);
    const BwdLayout l = bwd_layout_of(s);
    if (l.total && !workspace)
        return fail(SSD_ERR_NULL, "workspace is NULL (%zu bytes needed)", l.total);
    if (misaligned(workspace)) return fail(SSD_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (workspace_bytes < l.total)
        return fail(SSD_ERR_WORKSPACE, "workspace_bytes = %zu < %zu required", workspace_bytes,
                    l.total);
    if (s.Bt == 0) return ok();
    Ws w;
    if ((r = check_ws(s, workspace, workspace_bytes, &w)) != SSD_OK) return r;
    char *base = static_cast<char *>(workspace);
    float *fin = reinterpret_cast<float *>(base + l.fin);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the forward's chunk quantities again: G, DT, then h_prev in fp32 and the
    // final state, by the one-pass state stage where the forward would take
    // it, else by S (chunk_state) and state_passing, which writes fp32 h_prev
    // for fp32 io
    void *hp32 = s.bf16 ? static_cast<void *>(base + l.hp32) : w.hprev;
    // as in the forward, the one-pass recompute's B fragments come from the
    // cumsum's launch.  Where both scans take the one-pass form with the same
    // row split, they run as one grid (ssd::launch_state_pair); the adjoint
    // then writes ghat into the S region while the recompute still reads B
    // fragments, so these go to the C B^T region instead (written only after
    // both scans).
    const bool one_pass = bwd_one_pass(s);
    const bool adj_one_pass = one_pass && ssd::state_adj_supported(s);
    const int rows_f = state_fwd_rows() > 0 ? state_fwd_rows() : ssd::state_fwd_rows_per_block(s);
    const int rows_a = state_adj_rows() > 0 ? state_adj_rows() : ssd::state_adj_rows_per_block(s);
    const bool pair = adj_one_pass && rows_f == rows_a;
    void *bfrag = pair ? static_cast<void *>(base + l.cb3) : static_cast<void *>(w.S);
    if ((r = run_cumsum(s, dt, A, w, st, nullptr, one_pass ? B : nullptr, bfrag)) != SSD_OK)
        return r;
    if (pair) {
        r = hip_result(ssd::launch_state_pair(s, x, w.G, w.DT, init_state,
                                              static_cast<float *>(hp32), fin, bfrag,
                                              static_cast<const float *>(dy), C,
                                              static_cast<const float *>(dfinal), w.S,
                                              static_cast<float *>(dinit), base + l.cfr, rows_f,
                                              st),
                       "state_pair", st);
    } else if (one_pass) {
        r = hip_result(ssd::launch_state_fwd(s, x, B, w.G, w.DT, init_state, hp32, fin, w.S,
                                             state_fwd_rows(), true, st, true),
                       "state_fwd", st);
    } else {
        ssd::Shape s32 = s;
        s32.bf16 = false;
        if ((r = run_state(s, x, B, w, st)) != SSD_OK) return r;
        r = hip_result(ssd::launch_state_passing(s32, w.S, w.G, init_state, hp32, fin, st),
                       "state_passing", st);
    }
    if (r != SSD_OK) return r;
    ssd::BwdArgs a{x, B, C, A, D, dy, dfinal, fin, dinit, dx, ddt, dA, dB, dC, dD, w.G, w.DT,
                   w.S, hp32, s.bf16 ? nullptr : reinterpret_cast<float *>(base + l.cb),
                   reinterpret_cast<float *>(base + l.tok),
                   s.bf16 ? reinterpret_cast<uint16_t *>(base + l.cb3) : nullptr,
                   s.bf16 ? reinterpret_cast<uint16_t *>(base + l.cbt3) : nullptr,
                   s.bf16 ? reinterpret_cast<float *>(base + l.mt) : nullptr,
                   reinterpret_cast<double *>(base + l.part), false};
    // the state adjoint: the one-pass reverse scan where the forward takes the
    // one-pass form (run above when paired), else per-chunk sums and a
    // separate reverse scan
    if (pair) {
        a.ghat_ready = true;
    } else if (adj_one_pass) {
        r = hip_result(ssd::launch_state_adj(s, static_cast<const float *>(dy), C, w.G,
                                             static_cast<const float *>(dfinal), w.S,
                                             static_cast<float *>(dinit), base + l.cfr,
                                             state_adj_rows(), st),
                       "state_adj", st);
        if (r != SSD_OK) return r;
        a.ghat_ready = true;
    }
    r = hip_result(ssd::launch_chunked_bwd(s, a, st), "chunked_bwd", st);
    if (r != SSD_OK) return r;
    return ok();
}

const char *ssd_status_string(ssd_status status) {
    switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL: return "SSD_ERR_NULL: a required pointer is NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: a dimension is out of range";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: shape or dtype not instantiated";
    case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: pointer not 16-byte aligned";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace too small";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: a HIP call failed";
    }
    return "unknown ssd_status";
}

const char *ssd_last_error_detail(void) { return g_detail; }

int ssd_version(void) { return 100; }

}  // extern "C"
