// sv_api.hip -- the C ABI of libspecverify: argument checks, workspace layout,
// kernel launches on the caller's stream, and per-kernel event tracing.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "sv_device.hpp"
#include "sv_internal.hpp"
#include "sv_skip.hpp"

namespace sv {

RowGeom row_geom(int V, sv_dtype dt, bool ptrs_aligned, int vecs_per_lane) {
    RowGeom g;
    g.per_vec = dt == SV_BF16 ? 8 : 4;
    g.nvec = (V + g.per_vec - 1) / g.per_vec;
    const int per_wave = kWave * vecs_per_lane;
    g.segs = (g.nvec + per_wave - 1) / per_wave;
    if (g.segs < 1) g.segs = 1;
    g.ntiles = (g.nvec + kWave - 1) / kWave;
    g.aligned = ptrs_aligned && (V % g.per_vec) == 0;
    return g;
}

static size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

SampleWs sample_ws_layout(int B, int K, const RowGeom &g) {
    SampleWs w;
    const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(2 * K + 1);
    // partials of either pass: full read (g) or row skipping (its own segments)
    const int skip_segs = row_geom(g.nvec * g.per_vec, g.per_vec == 8 ? SV_BF16 : SV_F32, true,
                                   kSkipVecsPerLane * kSkipChunks).segs;
    const size_t parts = rows * static_cast<size_t>(std::max(g.segs, skip_segs));
    size_t o = 0;
    w.part_R = o;
    o = align_up(o + parts * sizeof(float));
    w.part_s = o;
    o = align_up(o + parts * sizeof(double));
    w.L2 = o;
    o = align_up(o + rows * sizeof(double));
    // the row-skipping pass clears part_R through the control words at once
    w.skipctl = o;
    o = align_up(o + skip_ctl_bytes(B, K));
    w.rp = o;
    o = align_up(o + static_cast<size_t>(B) * sizeof(ResidParam));
    w.tiles = o;
    o = align_up(o + static_cast<size_t>(B) * static_cast<size_t>(g.ntiles) * sizeof(double));
    w.total = o;
    return w;
}

int resid_tiles_per_wave(int B, int ntiles) {
    const long long total = static_cast<long long>(B) * ntiles;
    long long t = (total + kResidTargetWaves - 1) / kResidTargetWaves;
    t = ((t + kResidGroup - 1) / kResidGroup) * kResidGroup;
    return static_cast<int>(std::max<long long>(kResidGroup, std::min<long long>(t, 64)));
}

GreedyWs greedy_ws_layout(int B, int rows_per_req, const RowGeom &g) {
    GreedyWs w;
    // requests short enough for a row-skipping pass (chains of K <= 31, trees
    // of N <= 64) also hold that pass's keys, per-row argmax and control words
    const bool chain = skip_supported(rows_per_req - 1), tree = tree_skip_supported(rows_per_req);
    const bool skip = chain || tree;
    const int skip_segs = skip ? row_geom(g.nvec * g.per_vec, g.per_vec == 8 ? SV_BF16 : SV_F32, true,
                                          kGSkipVecsPerLane * kGSkipChunks).segs
                               : 0;
    const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(rows_per_req);
    size_t o = 0;
    w.part_k = o;
    o = align_up(o + rows * static_cast<size_t>(std::max(g.segs, skip_segs)) * sizeof(uint64_t));
    w.amax = o;
    if (skip) o = align_up(o + rows * sizeof(int32_t));
    w.skipctl = o;
    const size_t ctl = std::max(chain ? skip_ctl_bytes(B, rows_per_req - 1) + sizeof(unsigned) * B : 0,
                                tree ? tree_ctl_bytes(B, rows_per_req) : 0);
    if (skip) o = align_up(o + ctl);
    w.total = o;
    return w;
}

Scale make_scale(double T) {
    Scale s;
    s.c = 1.4426950408889634073599246810018921 / T;  // log2(e) / T
    float hi = static_cast<float>(s.c);
    if (static_cast<double>(hi) >= s.c) hi = nextafterf(hi, 0.0f);
    s.c_hi = hi;
    s.c_lo = static_cast<float>(s.c - static_cast<double>(hi));
    return s;
}

// ---- tracing ---------------------------------------------------------------------

namespace {
struct TraceRec {
    int kernel;
    hipEvent_t start, stop;
};
struct Tracer {
    std::mutex mu;
    bool on = false;
    int capacity = 0;
    int used = 0;
    unsigned mask = 0;
    std::vector<TraceRec> recs;
};
Tracer &tracer() {
    static Tracer t;
    return t;
}
// The kernel the calling thread launches next: per thread, so that host threads
// launching at the same time never label each other's launches.
thread_local int t_next_kernel = -1;

void destroy_events(std::vector<TraceRec> &recs) {
    for (auto &r : recs) {
        if (r.start) (void)hipEventDestroy(r.start);
        if (r.stop) (void)hipEventDestroy(r.stop);
    }
    recs.clear();
}
}  // namespace

void trace_select(int kernel) { t_next_kernel = kernel; }

bool trace_events(hipEvent_t *start, hipEvent_t *stop) {
    const int k = t_next_kernel;
    t_next_kernel = -1;
    Tracer &t = tracer();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.on || k < 0 || t.used >= t.capacity) return false;
    if (t.mask != 0 && !(t.mask & (1u << k))) return false;
    TraceRec &r = t.recs[t.used++];
    r.kernel = k;
    *start = r.start;
    *stop = r.stop;
    return true;
}

}  // namespace sv

using namespace sv;

namespace {

bool valid_dtype(sv_dtype dt) { return dt == SV_F32 || dt == SV_BF16; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// Every launch goes through here so tracing knows which kernel it is.
template <typename F>
hipError_t traced(int kernel, hipStream_t, F &&f) {
    trace_select(kernel);
    return f();
}

// Element counts must stay addressable with 64-bit offsets and int32 row lengths.
bool sizes_ok(long long B, long long rows_per_req, long long V) {
    if (B < 0 || rows_per_req < 0 || V < 1 || V > 0x7fffffffLL / 8) return false;
    const double elems = static_cast<double>(B) * static_cast<double>(rows_per_req) * static_cast<double>(V);
    return elems < 9.0e15;
}

}  // namespace

extern "C" {

size_t sv_sample_workspace_bytes(int B, int K, int V, sv_dtype dt) {
    if (B < 0 || K < 0 || K > SV_MAX_DRAFT_LEN || !valid_dtype(dt) || !sizes_ok(B, 2LL * K + 1, V)) return 0;
    const RowGeom g = row_geom(V, dt, true, kStatsVecsPerLane);
    return sample_ws_layout(B, K, g).total;
}

size_t sv_greedy_workspace_bytes(int B, int rows_per_req, int V, sv_dtype dt) {
    if (B < 0 || rows_per_req < 1 || !valid_dtype(dt) || !sizes_ok(B, rows_per_req, V)) return 0;
    const RowGeom g = row_geom(V, dt, true, kArgmaxVecsPerLane);
    return greedy_ws_layout(B, rows_per_req, g).total;
}

}  // extern "C"

namespace {

// Where a sample call's workspace comes from: the caller's buffer, or the
// library's own scratch array of the current device (resolved only after
// every host-side check has passed, so a rejected call touches no device).
struct WsSource {
    void *buf;
    size_t bytes;
    bool scratch;
};

sv_status device_scratch(void **out);

sv_status sample_impl(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                      const float *u_accept, const float *u_sample, int B, int K, int V, sv_dtype dt,
                      float temperature, int32_t *accept_len, int32_t *out_tokens, float *lse_target,
                      float *lse_draft, int32_t *req_status, WsSource src, hipStream_t stream) {
    if (!valid_dtype(dt)) return SV_ERR_UNSUPPORTED;
    if (B < 0 || K < 0 || V < 1 || !(temperature > 0.0f) || !isfinite(temperature))
        return SV_ERR_INVALID_ARG;
    if (K > SV_MAX_DRAFT_LEN || !sizes_ok(B, 2LL * K + 1, V)) return SV_ERR_UNSUPPORTED;
    if (B == 0) return SV_OK;
    if (!target_logits || !u_sample || !accept_len || !out_tokens || (!src.scratch && !src.buf))
        return SV_ERR_INVALID_ARG;
    if (K > 0 && (!draft_logits || !draft_tokens || !u_accept)) return SV_ERR_INVALID_ARG;
    if (!src.scratch && !aligned256(src.buf)) return SV_ERR_INVALID_ARG;
    const bool ptr_al = aligned16(target_logits) && (K == 0 || aligned16(draft_logits));
    const RowGeom g = row_geom(V, dt, ptr_al, kStatsVecsPerLane);
    const SampleWs L = sample_ws_layout(B, K, g);
    if (src.bytes < L.total) return src.scratch ? SV_ERR_SCRATCH : SV_ERR_WORKSPACE;
    if (src.scratch) {
        const sv_status st = device_scratch(&src.buf);
        if (st != SV_OK) return st;
    }

    char *ws = static_cast<char *>(src.buf);
    float *part_R = reinterpret_cast<float *>(ws + L.part_R);
    double *part_s = reinterpret_cast<double *>(ws + L.part_s);
    double *L2 = reinterpret_cast<double *>(ws + L.L2);
    ResidParam *rp = reinterpret_cast<ResidParam *>(ws + L.rp);
    double *tiles = reinterpret_cast<double *>(ws + L.tiles);
    const Scale sc = make_scale(static_cast<double>(temperature));
    if (!(sc.c < 0x1p127)) return SV_ERR_UNSUPPORTED;  // T below ~1e-38: log2(e)/T beyond fp32 range
    hipStream_t s = stream;
    const long long rows_t = static_cast<long long>(B) * (K + 1);
    const long long rows_total = rows_t + static_cast<long long>(B) * K;

    hipError_t e = hipSuccess;
    const RowGeom gs = row_geom(V, dt, ptr_al, kSkipVecsPerLane * kSkipChunks);
    if (lse_target || lse_draft || !skip_supported(K) ||
        !skip_grid_fits(static_cast<long long>(K + 1) * B * 2 * gs.segs, gs.segs)) {
        // every row is read (its statistics feed the lse outputs)
        e = traced(SV_K_ROWSTATS, s, [&] {
            return launch_rowstats(target_logits, draft_logits, rows_t, rows_total, V, g, dt, sc, part_R,
                                   part_s, s);
        });
        if (e == hipSuccess)
            e = traced(SV_K_ACCEPT, s, [&] {
                const PartRows pt{part_R, part_s, g.segs};
                const PartRows pd{part_R + rows_t * g.segs, part_s + rows_t * g.segs, g.segs};
                return launch_accept(target_logits, draft_logits, draft_tokens, u_accept, u_sample, B, K,
                                     V, dt, sc, pt, pd, nullptr, L2, accept_len, out_tokens, lse_target,
                                     lse_draft, req_status, rp, s);
            });
    } else {
        // rows of positions after each request's first rejection are not read
        e = launch_skip(target_logits, draft_logits, draft_tokens, u_accept, u_sample, B, K, V, gs, dt, sc,
                        part_R, part_s, L2, ws + L.skipctl, accept_len, out_tokens, req_status, rp, s);
    }
    if (e == hipSuccess)
        e = traced(SV_K_RESID_MASS, s, [&] {
            return launch_resid_mass(target_logits, draft_logits, B, V, g, dt, dt, sc, rp, tiles, s);
        });
    if (e == hipSuccess)
        e = traced(SV_K_RESID_SELECT, s, [&] {
            return launch_resid_select(target_logits, draft_logits, B, K, V, g, dt, dt, sc, rp, tiles,
                                       out_tokens, s);
        });
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace

// ---- the sampler's scratch for callers that cannot allocate ------------------------
//
// One array per device, loaded with the library's code object.  Host code
// never passes `scratch` itself to a kernel (on the host it names a stand-in,
// not device memory): each device's address comes from hipGetSymbolAddress,
// taken once with that device current and kept below.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];

sv_status device_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
    if (dev < 0 || dev >= kMaxScratchDevices) return SV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SV_OK;
}

}  // namespace

extern "C" {

sv_status spec_verify_sample(const void *target_logits, const void *draft_logits,
                             const int32_t *draft_tokens, const float *u_accept,
                             const float *u_sample, int B, int K, int V, sv_dtype dt,
                             float temperature, int32_t *accept_len, int32_t *out_tokens,
                             float *lse_target, float *lse_draft, int32_t *req_status,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return sample_impl(target_logits, draft_logits, draft_tokens, u_accept, u_sample, B, K, V, dt,
                       temperature, accept_len, out_tokens, lse_target, lse_draft, req_status,
                       WsSource{workspace, workspace_bytes, false}, stream);
}

sv_status spec_verify_sample_noalloc(const void *target_logits, const void *draft_logits,
                                     const int32_t *draft_tokens, const float *u_accept,
                                     const float *u_sample, int B, int K, int V, sv_dtype dt,
                                     float temperature, int32_t *accept_len, int32_t *out_tokens,
                                     float *lse_target, float *lse_draft, int32_t *req_status,
                                     hipStream_t stream) {
    return sample_impl(target_logits, draft_logits, draft_tokens, u_accept, u_sample, B, K, V, dt,
                       temperature, accept_len, out_tokens, lse_target, lse_draft, req_status,
                       WsSource{nullptr, SV_NOALLOC_SCRATCH_BYTES, true}, stream);
}

sv_status spec_verify_greedy(const void *target_logits, const int32_t *draft_tokens, int B, int K,
                             int V, sv_dtype dt, int32_t *accept_len, int32_t *out_tokens,
                             int32_t *req_status, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    if (!valid_dtype(dt)) return SV_ERR_UNSUPPORTED;
    if (B < 0 || K < 0 || V < 1) return SV_ERR_INVALID_ARG;
    if (K > SV_MAX_DRAFT_LEN || !sizes_ok(B, static_cast<long long>(K) + 1, V)) return SV_ERR_UNSUPPORTED;
    if (B == 0) return SV_OK;
    if (!target_logits || !accept_len || !out_tokens || !workspace) return SV_ERR_INVALID_ARG;
    if (K > 0 && !draft_tokens) return SV_ERR_INVALID_ARG;
    if (!aligned256(workspace)) return SV_ERR_INVALID_ARG;
    const RowGeom g = row_geom(V, dt, aligned16(target_logits), kArgmaxVecsPerLane);
    const long long rows = static_cast<long long>(B) * (K + 1);
    const GreedyWs L = greedy_ws_layout(B, K + 1, g);
    if (workspace_bytes < L.total) return SV_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    uint64_t *pk = reinterpret_cast<uint64_t *>(ws + L.part_k);
    hipStream_t s = stream;
    hipError_t e = hipSuccess;
    const RowGeom gs = row_geom(V, dt, aligned16(target_logits), kGSkipVecsPerLane * kGSkipChunks);
    if (SV_GREEDY_SKIP && skip_supported(K) &&
        skip_grid_fits(static_cast<long long>(K + 1) * B * gs.segs, gs.segs)) {
        // rows of positions after each request's first mismatch are not read
        e = launch_skip_match(target_logits, draft_tokens, B, K, V, gs, dt, pk,
                              reinterpret_cast<int32_t *>(ws + L.amax), ws + L.skipctl, accept_len,
                              out_tokens, req_status, s);
    } else {
        e = traced(SV_K_ARGMAX, s, [&] { return launch_argmax(target_logits, rows, V, g, dt, pk, s); });
        if (e == hipSuccess)
            e = traced(SV_K_MATCH, s, [&] {
                return launch_match(pk, draft_tokens, B, K, V, g, accept_len, out_tokens, req_status, s);
            });
    }
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status spec_verify_tree(const void *target_logits, const int32_t *node_tokens,
                           const int32_t *parents, int B, int N, int V, sv_dtype dt,
                           int32_t *accept_len, int32_t *path_nodes, int32_t *out_tokens,
                           int32_t *req_status, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    if (!valid_dtype(dt)) return SV_ERR_UNSUPPORTED;
    if (B < 0 || N < 1 || V < 1) return SV_ERR_INVALID_ARG;
    if (N > SV_MAX_TREE_NODES || !sizes_ok(B, N, V)) return SV_ERR_UNSUPPORTED;
    if (B == 0) return SV_OK;
    if (!target_logits || !node_tokens || !parents || !accept_len || !path_nodes || !out_tokens ||
        !workspace)
        return SV_ERR_INVALID_ARG;
    if (!aligned256(workspace)) return SV_ERR_INVALID_ARG;
    const RowGeom g = row_geom(V, dt, aligned16(target_logits), kArgmaxVecsPerLane);
    const long long rows = static_cast<long long>(B) * N;
    const GreedyWs L = greedy_ws_layout(B, N, g);
    if (workspace_bytes < L.total) return SV_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    uint64_t *pk = reinterpret_cast<uint64_t *>(ws + L.part_k);
    hipStream_t s = stream;
    hipError_t e = hipSuccess;
    const RowGeom gs = row_geom(V, dt, aligned16(target_logits), kGSkipVecsPerLane * kGSkipChunks);
    if (SV_GREEDY_SKIP && tree_skip_supported(N) &&
        skip_grid_fits(static_cast<long long>(N) * B * gs.segs, gs.segs)) {
        // rows of rejected nodes are not read
        e = launch_skip_tree(target_logits, node_tokens, parents, B, N, V, gs, dt, pk,
                             reinterpret_cast<int32_t *>(ws + L.amax), ws + L.skipctl, accept_len, path_nodes,
                             out_tokens, req_status, s);
    } else {
        e = traced(SV_K_ARGMAX, s, [&] { return launch_argmax(target_logits, rows, V, g, dt, pk, s); });
        if (e == hipSuccess)
            e = traced(SV_K_TREE, s, [&] {
                return launch_tree(pk, node_tokens, parents, B, N, V, g, accept_len, path_nodes,
                                   out_tokens, req_status, s);
            });
    }
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

// ---- greedy verification fused with the LM-head projection ----------------------

static bool lmhead_sizes_ok(long long rows, int D, int V) {
    // element offsets of H and W rows stay within int32 inside the kernel
    return rows >= 1 && V >= 1 && D >= 128 && D % 128 == 0 && rows * (D / 8) < 0x7fffffffLL &&
           static_cast<long long>(V) * (D / 8) < 0x7fffffffLL;
}

size_t sv_lmhead_workspace_bytes(int rows, int V) {
    if (rows < 1 || V < 1) return 0;
    return align_up(static_cast<size_t>(rows) * static_cast<size_t>(lmhead_segs(V)) * sizeof(uint64_t));
}

static RowGeom lmhead_geom(int V) {
    RowGeom g;
    g.per_vec = 8;
    g.nvec = (V + 7) / 8;
    g.segs = lmhead_segs(V);
    g.ntiles = 0;
    g.aligned = true;
    return g;
}

sv_status spec_verify_greedy_lmhead(const void *hidden, const void *lm_head,
                                    const int32_t *draft_tokens, int B, int K, int D, int V,
                                    int32_t *accept_len, int32_t *out_tokens, int32_t *req_status,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || K < 0 || V < 1 || D < 1) return SV_ERR_INVALID_ARG;
    if (K > SV_MAX_DRAFT_LEN) return SV_ERR_UNSUPPORTED;
    if (B == 0) return SV_OK;
    const long long rows = static_cast<long long>(B) * (K + 1);
    if (!lmhead_sizes_ok(rows, D, V)) return SV_ERR_UNSUPPORTED;
    if (!hidden || !lm_head || !accept_len || !out_tokens || !workspace) return SV_ERR_INVALID_ARG;
    if (K > 0 && !draft_tokens) return SV_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(lm_head) || !aligned256(workspace)) return SV_ERR_INVALID_ARG;
    if (workspace_bytes < sv_lmhead_workspace_bytes(static_cast<int>(rows), V)) return SV_ERR_WORKSPACE;
    uint64_t *pk = static_cast<uint64_t *>(workspace);
    hipStream_t s = stream;
    hipError_t e = traced(SV_K_LMHEAD, s, [&] {
        return launch_lmhead_argmax(hidden, lm_head, static_cast<int>(rows), D, V, pk, s);
    });
    if (e == hipSuccess)
        e = traced(SV_K_MATCH, s, [&] {
            return launch_match(pk, draft_tokens, B, K, V, lmhead_geom(V), accept_len, out_tokens,
                                req_status, s);
        });
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status spec_verify_tree_lmhead(const void *hidden, const void *lm_head,
                                  const int32_t *node_tokens, const int32_t *parents, int B, int N,
                                  int D, int V, int32_t *accept_len, int32_t *path_nodes,
                                  int32_t *out_tokens, int32_t *req_status, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || N < 1 || V < 1 || D < 1) return SV_ERR_INVALID_ARG;
    if (N > SV_MAX_TREE_NODES) return SV_ERR_UNSUPPORTED;
    if (B == 0) return SV_OK;
    const long long rows = static_cast<long long>(B) * N;
    if (!lmhead_sizes_ok(rows, D, V)) return SV_ERR_UNSUPPORTED;
    if (!hidden || !lm_head || !node_tokens || !parents || !accept_len || !path_nodes || !out_tokens ||
        !workspace)
        return SV_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(lm_head) || !aligned256(workspace)) return SV_ERR_INVALID_ARG;
    if (workspace_bytes < sv_lmhead_workspace_bytes(static_cast<int>(rows), V)) return SV_ERR_WORKSPACE;
    uint64_t *pk = static_cast<uint64_t *>(workspace);
    hipStream_t s = stream;
    hipError_t e = traced(SV_K_LMHEAD, s, [&] {
        return launch_lmhead_argmax(hidden, lm_head, static_cast<int>(rows), D, V, pk, s);
    });
    if (e == hipSuccess)
        e = traced(SV_K_TREE, s, [&] {
            return launch_tree(pk, node_tokens, parents, B, N, V, lmhead_geom(V), accept_len, path_nodes,
                               out_tokens, req_status, s);
        });
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"

// ---- speculative sampling fused with the LM-head projection ----------------------

namespace {
struct SampleLmWs {
    size_t part_Rt, part_st, row_R, row_s, xlog, part_Rd, part_sd, L2, rp, rows_p, tiles, total;
};
// gd: the draft rows' streaming geometry; gr: the fp32 rows the draw reads.
SampleLmWs sample_lm_ws_layout(int B, int K, int V, const RowGeom &gd, const RowGeom &gr) {
    SampleLmWs w;
    const size_t rows_t = static_cast<size_t>(B) * (K + 1), rows_d = static_cast<size_t>(B) * K;
    const size_t pt = rows_t * static_cast<size_t>(lmhead_segs(V)), pd = rows_d * static_cast<size_t>(gd.segs);
    const size_t row_bytes = static_cast<size_t>(V) * sizeof(float);
    size_t o = 0;
    w.part_Rt = o;
    o = align_up(o + pt * sizeof(float));
    w.part_st = o;
    o = align_up(o + pt * sizeof(double));
    w.row_R = o;
    o = align_up(o + rows_t * sizeof(float));
    w.row_s = o;
    o = align_up(o + rows_t * sizeof(double));
    w.xlog = o;
    o = align_up(o + rows_t * sizeof(float));
    w.part_Rd = o;
    o = align_up(o + pd * sizeof(float));
    w.part_sd = o;
    o = align_up(o + pd * sizeof(double));
    w.L2 = o;
    o = align_up(o + static_cast<size_t>(B) * (2 * K + 1) * sizeof(double));
    w.rp = o;
    o = align_up(o + static_cast<size_t>(B) * sizeof(ResidParam));
    w.rows_p = o;
    o = align_up(o + static_cast<size_t>(B) * row_bytes);
    w.tiles = o;
    o = align_up(o + static_cast<size_t>(B) * static_cast<size_t>(gr.ntiles) * sizeof(double));
    w.total = o;
    return w;
}
}  // namespace

extern "C" {

size_t sv_sample_lmhead_workspace_bytes(int B, int K, int D, int V, sv_dtype dt) {
    if (B < 1 || K < 0 || K > SV_MAX_DRAFT_LEN || !valid_dtype(dt) || V < 1 ||
        !lmhead_sizes_ok(static_cast<long long>(B) * (K + 1), D, V) || !sizes_ok(B, 2LL * K + 1, V))
        return 0;
    const RowGeom gd = row_geom(V, dt, true, kStatsVecsPerLane);
    const RowGeom gr = row_geom(V, SV_F32, true, kStatsVecsPerLane);
    return sample_lm_ws_layout(B, K, V, gd, gr).total;
}

sv_status spec_verify_sample_lmhead(const void *hidden, const void *lm_head, const void *draft_logits,
                                    const int32_t *draft_tokens, const float *u_accept,
                                    const float *u_sample, int B, int K, int D, int V, sv_dtype dt,
                                    float temperature, int32_t *accept_len, int32_t *out_tokens,
                                    float *lse_target, float *lse_draft, int32_t *req_status,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dtype(dt)) return SV_ERR_UNSUPPORTED;
    if (B < 0 || K < 0 || V < 1 || D < 1 || !(temperature > 0.0f) || !isfinite(temperature))
        return SV_ERR_INVALID_ARG;
    if (K > SV_MAX_DRAFT_LEN) return SV_ERR_UNSUPPORTED;
    if (B == 0) return SV_OK;
    const long long rows_t = static_cast<long long>(B) * (K + 1);
    if (!lmhead_sizes_ok(rows_t, D, V) || !sizes_ok(B, 2LL * K + 1, V)) return SV_ERR_UNSUPPORTED;
    if (!hidden || !lm_head || !u_sample || !accept_len || !out_tokens || !workspace)
        return SV_ERR_INVALID_ARG;
    if (K > 0 && (!draft_logits || !draft_tokens || !u_accept)) return SV_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(lm_head) || !aligned256(workspace)) return SV_ERR_INVALID_ARG;
    const RowGeom gd = row_geom(V, dt, K == 0 || aligned16(draft_logits), kStatsVecsPerLane);
    const RowGeom gr = row_geom(V, SV_F32, true, kStatsVecsPerLane);
    const SampleLmWs L = sample_lm_ws_layout(B, K, V, gd, gr);
    if (workspace_bytes < L.total) return SV_ERR_WORKSPACE;
    const Scale sc = make_scale(static_cast<double>(temperature));
    if (!(sc.c < 0x1p127)) return SV_ERR_UNSUPPORTED;

    char *ws = static_cast<char *>(workspace);
    float *part_Rt = reinterpret_cast<float *>(ws + L.part_Rt);
    double *part_st = reinterpret_cast<double *>(ws + L.part_st);
    float *row_R = reinterpret_cast<float *>(ws + L.row_R);
    double *row_s = reinterpret_cast<double *>(ws + L.row_s);
    float *xlog = reinterpret_cast<float *>(ws + L.xlog);
    float *part_Rd = reinterpret_cast<float *>(ws + L.part_Rd);
    double *part_sd = reinterpret_cast<double *>(ws + L.part_sd);
    double *L2 = reinterpret_cast<double *>(ws + L.L2);
    ResidParam *rp = reinterpret_cast<ResidParam *>(ws + L.rp);
    float *rows_p = reinterpret_cast<float *>(ws + L.rows_p);
    double *tiles = reinterpret_cast<double *>(ws + L.tiles);
    hipStream_t s = stream;

    // 1. target rows: partials and the logit at each draft, from H W^T
    hipError_t e = traced(SV_K_LMHEAD_STATS, s, [&] {
        return launch_lmhead_stats(hidden, lm_head, B, K, D, V, draft_tokens, sc, part_Rt, part_st, xlog, s);
    });
    // 2. the target rows' partials merged to one per row; the draft rows'
    //    partials from the streaming statistics pass
    if (e == hipSuccess)
        e = traced(SV_K_MERGE_PARTS, s, [&] {
            return launch_merge_parts(part_Rt, part_st, rows_t, lmhead_segs(V), row_R, row_s, s);
        });
    if (e == hipSuccess && K > 0)
        e = traced(SV_K_ROWSTATS, s, [&] {
            return launch_rowstats(nullptr, draft_logits, 0, static_cast<long long>(B) * K, V, gd, dt, sc,
                                   part_Rd, part_sd, s);
        });
    // 3. merge, acceptance scan, lse outputs, draw parameters
    if (e == hipSuccess)
        e = traced(SV_K_ACCEPT, s, [&] {
            const PartRows pt{row_R, row_s, 1};
            const PartRows pd{part_Rd, part_sd, gd.segs};
            return launch_accept(nullptr, draft_logits, draft_tokens, u_accept, u_sample, B, K, V, dt, sc, pt,
                                 pd, xlog, L2, accept_len, out_tokens, lse_target, lse_draft, req_status, rp, s);
        });
    // 4. the row each request draws from, formed again and written in fp32
    if (e == hipSuccess)
        e = traced(SV_K_LMHEAD_ROWS, s,
                   [&] { return launch_lmhead_rows(hidden, lm_head, B, K, D, V, rp, rows_p, s); });
    // 5. the draw, beside the draft row read where it lies
    if (e == hipSuccess)
        e = traced(SV_K_RESID_MASS, s, [&] {
            return launch_resid_mass(rows_p, draft_logits, B, V, gr, SV_F32, dt, sc, rp, tiles, s);
        });
    if (e == hipSuccess)
        e = traced(SV_K_RESID_SELECT, s, [&] {
            return launch_resid_select(rows_p, draft_logits, B, K, V, gr, SV_F32, dt, sc, rp, tiles, out_tokens,
                                       s);
        });
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"

// ---- AdaPLD lexical retrieval ----------------------------------------------------

extern "C" {


size_t sv_ngram_workspace_bytes(int B, int L) {
    if (B < 0 || L < 1) return 0;
    return align_up(static_cast<size_t>(B) * static_cast<size_t>(ngram_chunks(L)) * sizeof(int32_t));
}

sv_status spec_ngram_candidates(const int32_t *context, int B, int L, const int32_t *lengths,
                                const int32_t *queries, int n, int cap, int32_t *count,
                                int32_t *positions, int32_t *req_status, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || L < 1 || n < 1 || cap < 0) return SV_ERR_INVALID_ARG;
    if (n > 64 || static_cast<long long>(B) * ngram_chunks(L) > 0x7fffffffLL) return SV_ERR_UNSUPPORTED;
    if (B == 0) return SV_OK;
    if (!context || !lengths || !queries || !count || (cap > 0 && !positions) || !workspace)
        return SV_ERR_INVALID_ARG;
    if (!aligned256(workspace)) return SV_ERR_INVALID_ARG;
    if (workspace_bytes < sv_ngram_workspace_bytes(B, L)) return SV_ERR_WORKSPACE;
    hipStream_t s = stream;
    const hipError_t e = launch_ngram(context, B, L, lengths, queries, n, cap, static_cast<int32_t *>(workspace),
                                      count, positions, req_status, s);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status spec_commit_tree_kv(const void *src_kv, void *dst_kv, int G, int B, int S, int row_bytes,
                              const int32_t *tree_base, const int32_t *commit_base,
                              const int32_t *accept_len, const int32_t *path_nodes, int N,
                              int32_t *req_status, hipStream_t stream) {
    if (G < 1 || B < 0 || S < 1 || N < 1 || row_bytes < 16 || row_bytes % 16 != 0)
        return SV_ERR_INVALID_ARG;
    if (N > SV_MAX_TREE_NODES || static_cast<long long>(G) * B > 0x7fffffffLL ||
        static_cast<long long>(N) * (row_bytes / 16) > 0x7fffffffLL)
        return SV_ERR_UNSUPPORTED;
    const double bytes = static_cast<double>(G) * B * static_cast<double>(S) * row_bytes;
    if (bytes >= 9.0e18) return SV_ERR_UNSUPPORTED;
    if (B == 0) return SV_OK;
    if (!src_kv || !dst_kv || !tree_base || !commit_base || !accept_len || !path_nodes)
        return SV_ERR_INVALID_ARG;
    if (!aligned16(src_kv) || !aligned16(dst_kv)) return SV_ERR_INVALID_ARG;
    hipStream_t s = stream;
    const hipError_t e = traced(SV_K_COMMIT, s, [&] {
        return launch_commit(src_kv, dst_kv, G, B, S, row_bytes, tree_base, commit_base, accept_len,
                             path_nodes, N, req_status, s);
    });
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

size_t sv_read_probe_folds(size_t bytes) {
    return static_cast<size_t>(read_probe_waves(static_cast<long long>(bytes / 16)));
}

sv_status sv_read_probe(const void *buf, size_t bytes, unsigned *folds, hipStream_t stream) {
    if (bytes % 16 != 0) return SV_ERR_INVALID_ARG;
    if (bytes / 16 > (1ull << 40)) return SV_ERR_UNSUPPORTED;
    if (bytes == 0) return SV_OK;
    if (!buf || !folds || !aligned16(buf)) return SV_ERR_INVALID_ARG;
    hipStream_t s = stream;
    const hipError_t e = traced(SV_K_READ_PROBE, s, [&] {
        return launch_read_probe(buf, static_cast<long long>(bytes / 16), folds, s);
    });
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

const char *sv_status_string(sv_status st) {
    switch (st) {
        case SV_OK: return "ok";
        case SV_ERR_INVALID_ARG: return "invalid argument";
        case SV_ERR_UNSUPPORTED: return "unsupported dtype or size";
        case SV_ERR_WORKSPACE: return "workspace too small";
        case SV_ERR_HIP: return "HIP runtime error";
        case SV_ERR_SCRATCH: return "sizes need more than the library's static scratch";
        default: break;
    }
    return "unknown status";
}

const char *sv_version(void) { return "specverify 0.1.0 (gfx950)"; }

const char *sv_kernel_name(int k) {
    static const char *names[SV_K_COUNT] = {"rowstats", "accept", "resid_mass", "resid_select",
                                            "argmax", "match", "tree", "skip_stats",
                                            "skip_argmax", "commit", "lmhead", "ngram_count",
                                            "ngram_emit", "skip_tree", "read_probe", "lmhead_stats",
                                            "lmhead_rows", "merge_parts"};
    return (k >= 0 && k < SV_K_COUNT) ? names[k] : "unknown";
}

sv_status sv_trace_begin(int capacity, unsigned kernel_mask) {
    if (capacity < 1) return SV_ERR_INVALID_ARG;
    Tracer &t = tracer();
    std::lock_guard<std::mutex> g(t.mu);
    destroy_events(t.recs);
    t.on = false;
    t.used = t.capacity = 0;
    t.recs.assign(static_cast<size_t>(capacity), TraceRec{-1, nullptr, nullptr});
    for (auto &r : t.recs) {
        if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) {
            destroy_events(t.recs);
            return SV_ERR_HIP;
        }
    }
    t.capacity = capacity;
    t.mask = kernel_mask;
    t.on = true;
    return SV_OK;
}

int sv_trace_end(sv_kernel_time *records, int max_records) {
    Tracer &t = tracer();
    std::lock_guard<std::mutex> g(t.mu);
    const int n = t.used;
    for (int i = 0; i < n; ++i) {
        float ms = -1.0f;
        if (hipEventSynchronize(t.recs[i].stop) == hipSuccess)
            (void)hipEventElapsedTime(&ms, t.recs[i].start, t.recs[i].stop);
        if (records && i < max_records) records[i] = sv_kernel_time{t.recs[i].kernel, ms};
    }
    destroy_events(t.recs);
    t.on = false;
    t.used = t.capacity = 0;
    return n;
}

}  // extern "C"
