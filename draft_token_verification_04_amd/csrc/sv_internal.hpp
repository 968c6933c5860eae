// sv_internal.hpp -- host-side geometry, workspace layout and kernel launchers
// shared by the C-ABI entry points and the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
#ifndef SV_STATS_VECS
#define SV_STATS_VECS 16
#endif
#ifndef SV_ARGMAX_VECS
#define SV_ARGMAX_VECS 8
#endif
#ifndef SV_RESID_GROUP
#define SV_RESID_GROUP 2
#endif
#ifndef SV_SKIP_VECS
#define SV_SKIP_VECS 6
#endif
#ifndef SV_SKIP_CHUNKS
#define SV_SKIP_CHUNKS 2
#endif
// Greedy chains with K <= 31 take the row-skipping pass (0: always read every row).
#ifndef SV_GREEDY_SKIP
#define SV_GREEDY_SKIP 1
#endif
// 16-byte vectors per lane held in registers by one streaming wave of the
// row-statistics and argmax passes (a wave covers 64 * this many vectors).
constexpr int kStatsVecsPerLane = SV_STATS_VECS;
constexpr int kArgmaxVecsPerLane = SV_ARGMAX_VECS;
// Tiles (64 vectors each) loaded together by the residual-mass pass; a wave
// walks its tiles in such groups, loading the next group before summing one.
constexpr int kResidGroup = SV_RESID_GROUP;
// The row-skipping pass: a wave streams SV_SKIP_CHUNKS chunks of
// SV_SKIP_VECS vectors per lane, loading each chunk while it sums the last.
// Measured on MI355X (us per pass, B = 256 / B = 32, K = 7, V = 151936 bf16):
// 6 x 2 (12 KB per wave) 93.9 / 31.6; 6 x 3 93.5 / 33.4; 4 x 3 94.7 / 33.3;
// 8 x 2 99.2 / -; 8 x 4 103.6 / -; 12 x 1 99.5 / 30.3; 4 x 6 102.6 / 35.3.
constexpr int kSkipVecsPerLane = SV_SKIP_VECS;
constexpr int kSkipChunks = SV_SKIP_CHUNKS;
// The same shape for the greedy chain's row-skipping pass (its waves are best
// kept short: a position's segments then finish, and its decisions land,
// sooner, so fewer rows past each mismatch are read).
#ifndef SV_GSKIP_VECS
#define SV_GSKIP_VECS 8
#endif
#ifndef SV_GSKIP_CHUNKS
#define SV_GSKIP_CHUNKS 2
#endif
constexpr int kGSkipVecsPerLane = SV_GSKIP_VECS;
// Dynamic LDS each workgroup of the greedy chain's and the tree's skip passes
// reserves, unused, to cap the workgroups per compute unit (0: as many as their
// registers allow, five).  Measured on MI355X (us per pass, chain B=256 / chain
// B=512 / tree B=64), in plain request order: no cap 69.6 / 116.1 / 70.0;
// 40 KB (four) 67.4 / 111.1 / 71.9; 45 KB (three) 68.1 / 115.8 / 77.5; 54 KB
// (two) 75.6 / 143.8 / 92.9.  With the rotated orders (skip_request): chain
// 32 KB / 40 KB / 52 KB 64.4 / 64.4 / 64.5 (B=256), 109.2 / 109.1 / 111.9
// (B=512); tree no cap 70.3-70.7, 40 KB 67.7-68.0, 32 KB 68.0, 24 KB 69.6,
// 20 KB 69.8.
#ifndef SV_GSKIP_LDS
#define SV_GSKIP_LDS (40 * 1024)
#endif
#ifndef SV_TSKIP_LDS
#define SV_TSKIP_LDS (40 * 1024)
#endif
// Bound on any poll of a word another wave is bound to write (never reached).
constexpr int kSkipPollCap = 1 << 22;

constexpr int kGSkipChunks = SV_GSKIP_CHUNKS;
// Waves the residual-mass pass aims for: short waves of a few tiles each.
// Measured on MI355X at B=256 (V=151936 bf16, rows evicted before each call,
// as they are after the statistics pass): 49152 (one group of 2 tiles per
// wave) 24.9-25.0 us, 32768 (4 tiles) 26.0-26.2, 16384 (6 tiles) 26.2, and
// one tile per wave 27.4-28.8; 4096 longer waves ran 32 us.
#ifndef SV_RESID_WAVES
#define SV_RESID_WAVES 49152
#endif
constexpr int kResidTargetWaves = SV_RESID_WAVES;
// Bytes of LDS the per-request merge kernels use to stage row partials.
constexpr int kMergeLdsBytes = 24 * 1024;

// How one row of V logits is cut into per-wave segments.
struct RowGeom {
    int per_vec;   // elements per 16-byte vector (4 for f32, 8 for bf16)
    int nvec;      // vectors per row: ceil(V / per_vec)
    int segs;      // segments (one wave each) per row
    int ntiles;    // 64-vector tiles per row (residual pass)
    bool aligned;  // 16-byte loads (rows 16-byte aligned, V % per_vec == 0)
};

RowGeom row_geom(int V, sv_dtype dt, bool ptrs_aligned, int vecs_per_lane);

// Parameters of the one token drawn per request, written by the acceptance
// kernel and read by the residual kernels.
struct ResidParam {
    double L2p;    // log2 sum_v 2^(Lp[v] c) of the target row
    double L2q;    // same for the draft row (pair mode only)
    double u;      // the uniform for this draw
    long long row_p;  // global target row index
    long long row_q;  // global draft row index (pair mode only)
    int mode;      // 1 = residual max(0, p - q), 0 = p alone (bonus)
    int pos;       // output slot n (= accept_len)
    // The draw's per-row constants: with R = L2 + 1 split as R_hi + R_lo
    // (R_hi the nearest float), Rp_hi and Rq_hi for the two rows, and
    // r = 2^(Rq_lo - Rp_lo) (1 for the bonus).
    float Rp_hi, Rq_hi, r;
};

// Byte offsets of the workspace regions.
struct SampleWs {
    size_t part_R, part_s, L2, rp, tiles, skipctl, total;
};
struct GreedyWs {
    size_t part_k, amax, skipctl, total;  // amax/skipctl: chains of K <= 31 only
};
SampleWs sample_ws_layout(int B, int K, const RowGeom &g);
int resid_tiles_per_wave(int B, int ntiles);
GreedyWs greedy_ws_layout(int B, int rows_per_req, const RowGeom &g);

// Temperature scale c = log2(e)/T split as c_hi + c_lo with both floats and
// c_lo > 0, so x*c_hi + x*c_lo reproduces x*c to ~2^-48 and -inf*c stays -inf.
struct Scale {
    double c;
    float c_hi, c_lo;
};
Scale make_scale(double T);

// Kernel-launch tracing.  trace_select() names the kernel the next launch is;
// trace_events() hands out the event pair that launch should carry (false when
// tracing is off, full, or masked for that kernel).
void trace_select(int kernel);
bool trace_events(hipEvent_t *start, hipEvent_t *stop);

// Launch `k` on `s`; when tracing claims it, the launch carries start/stop
// events stamped by the dispatch itself (hipExtLaunchKernelGGL).
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*k)(KArgs...), dim3 grid, dim3 block, size_t lds,
                                hipStream_t s, Args... args) {
    hipEvent_t e0, e1;
    if (trace_events(&e0, &e1))
        hipExtLaunchKernelGGL(k, grid, block, static_cast<uint32_t>(lds), s, e0, e1, 0u,
                              static_cast<KArgs>(args)...);
    else
        hipLaunchKernelGGL(k, grid, block, lds, s, static_cast<KArgs>(args)...);
    return hipGetLastError();
}

// ---- launchers (each enqueues one kernel on `s`) --------------------------------
hipError_t launch_rowstats(const void *tgt, const void *drf, long long rows_t, long long rows_total,
                           int V, const RowGeom &g, sv_dtype dt, const Scale &sc, float *part_R,
                           double *part_s, hipStream_t s);
// Segment partials (R, s) of a set of rows, `segs` per row, row-major.
struct PartRows {
    const float *R;
    const double *s;
    int segs;
};
// Merge, acceptance scan and draw parameters.  pt holds the B (K+1) target
// rows' partials and pd the B K draft rows'.  xlog non-null selects the fused
// form: the target logit at each draft is read from xlog [B (K+1)] instead of
// the target rows (tgt is then unused), and the draw's rows are numbered per
// request (row b of the buffers the draw reads).
hipError_t launch_accept(const void *tgt, const void *drf, const int32_t *drafts, const float *ua,
                         const float *us, int B, int K, int V, sv_dtype dt, const Scale &sc,
                         const PartRows &pt, const PartRows &pd, const float *xlog, double *L2,
                         int32_t *accept_len, int32_t *out_tokens, float *lse_t, float *lse_d,
                         int32_t *status, ResidParam *rp, hipStream_t s);
bool skip_supported(int K);
size_t skip_ctl_bytes(int B, int K);
hipError_t launch_skip(const void *tgt, const void *drf, const int32_t *drafts, const float *ua,
                       const float *us, int B, int K, int V, const RowGeom &g, sv_dtype dt,
                       const Scale &sc, float *part_R, double *part_s, double *L2, void *ctl_base,
                       int32_t *accept_len, int32_t *out_tokens, int32_t *status, ResidParam *rp,
                       hipStream_t s);
// dt: the target rows' type (g is their geometry); dq: the draft rows' type,
// equal to dt or bf16 beside fp32 target rows.
hipError_t launch_resid_mass(const void *tgt, const void *drf, int B, int V, const RowGeom &g,
                             sv_dtype dt, sv_dtype dq, const Scale &sc, const ResidParam *rp,
                             double *tile_mass, hipStream_t s);
hipError_t launch_resid_select(const void *tgt, const void *drf, int B, int K, int V,
                               const RowGeom &g, sv_dtype dt, sv_dtype dq, const Scale &sc,
                               const ResidParam *rp, double *tile_mass, int32_t *out_tokens,
                               hipStream_t s);
hipError_t launch_argmax(const void *L, long long rows, int V, const RowGeom &g, sv_dtype dt,
                         uint64_t *part_k, hipStream_t s);
hipError_t launch_skip_match(const void *L, const int32_t *drafts, int B, int K, int V,
                             const RowGeom &g, sv_dtype dt, uint64_t *part_k, int32_t *amax,
                             void *ctl_base, int32_t *accept_len, int32_t *out_tokens,
                             int32_t *status, hipStream_t s);
int ngram_chunks(int L);
hipError_t launch_ngram(const int32_t *ctx, int B, int L, const int32_t *lens, const int32_t *queries,
                        int n, int cap, int32_t *counts, int32_t *count, int32_t *positions,
                        int32_t *status, hipStream_t s);
int lmhead_segs(int V);
hipError_t launch_lmhead_argmax(const void *H, const void *W, int M, int D, int V, uint64_t *part_k,
                                hipStream_t s);
// Rows b (K+1) + i of H [B (K+1)][D] projected on W [V][D]: per row and
// 128-column segment the (R, s) partials at scale sc, and in xlog the logit at
// draft i (drafts [B][K]) for i < K.
hipError_t launch_lmhead_stats(const void *H, const void *W, int B, int K, int D, int V,
                               const int32_t *drafts, const Scale &sc, float *part_R, double *part_s,
                               float *xlog, hipStream_t s);
// Row b of rows [B][V] (fp32) = the logits of H row b (K+1) + rp[b].pos.
hipError_t launch_lmhead_rows(const void *H, const void *W, int B, int K, int D, int V,
                              const ResidParam *rp, float *rows, hipStream_t s);
// One (R, s) partial per row out of `segs` per row (the merge k_accept does,
// so that merging the single partial gives the same normaliser bit for bit).
hipError_t launch_merge_parts(const float *R, const double *S, long long rows, int segs, float *outR,
                              double *outS, hipStream_t s);
hipError_t launch_commit(const void *src, void *dst, int G, int B, int S, int row_bytes,
                         const int32_t *tree_base, const int32_t *commit_base,
                         const int32_t *accept_len, const int32_t *path_nodes, int N,
                         int32_t *status, hipStream_t s);
// Zeroes `bytes` (a multiple of 4) at `base` with an untraced launch.
hipError_t clear_words(void *base, size_t bytes, hipStream_t s);
bool tree_skip_supported(int N);
size_t tree_ctl_bytes(int B, int N);
long long read_probe_waves(long long n16);
hipError_t launch_read_probe(const void *buf, long long n16, unsigned *folds, hipStream_t s);
hipError_t launch_skip_tree(const void *L, const int32_t *node_tokens, const int32_t *parents, int B, int N,
                            int V, const RowGeom &g, sv_dtype dt, uint64_t *part_k, int32_t *amax,
                            void *ctl_base, int32_t *accept_len, int32_t *path_nodes, int32_t *out_tokens,
                            int32_t *status, hipStream_t s);
hipError_t launch_match(const uint64_t *part_k, const int32_t *drafts, int B, int K, int V,
                        const RowGeom &g, int32_t *accept_len, int32_t *out_tokens, int32_t *status,
                        hipStream_t s);
hipError_t launch_tree(const uint64_t *part_k, const int32_t *node_tokens,
                       const int32_t *parents, int B, int N, int V, const RowGeom &g,
                       int32_t *accept_len, int32_t *path_nodes, int32_t *out_tokens,
                       int32_t *status, hipStream_t s);

}  // namespace sv
