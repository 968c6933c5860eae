// sv_internal.hpp -- host-side geometry, workspace layout and kernel launchers
// shared by the C-ABI entry points and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

// 16-byte vectors per lane held in registers by one streaming wave.
constexpr int kStreamVecsPerLane = 8;
// Tiles (64 vectors each) per wave in the residual-mass pass.
constexpr int kTilesPerWave = 8;
// Longest draft chain accepted by spec_verify_sample (row statistics of one
// request are kept in LDS by the acceptance kernel).
constexpr int kMaxSampleK = 1024;

// How one row of V logits is cut into per-wave segments.
struct RowGeom {
    int per_vec;   // elements per 16-byte vector (4 for f32, 8 for bf16)
    int nvec;      // vectors per row: ceil(V / per_vec)
    int segs;      // segments (one wave each) per row
    int ntiles;    // 64-vector tiles per row (residual pass)
    bool aligned;  // 16-byte loads (rows 16-byte aligned, V % per_vec == 0)
};

RowGeom row_geom(int V, sv_dtype dt, bool ptrs_aligned);

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
};

// Byte offsets of the workspace regions.
struct SampleWs {
    size_t part_R, part_s, L2, rp, tiles, total;
};
struct GreedyWs {
    size_t part_v, part_i, total;
};
SampleWs sample_ws_layout(int B, int K, const RowGeom &g);
GreedyWs greedy_ws_layout(long long rows, const RowGeom &g);

// Temperature scale c = log2(e)/T split as c_hi + c_lo with both floats and
// c_lo > 0, so x*c_hi + x*c_lo reproduces x*c to ~2^-48 and -inf*c stays -inf.
struct Scale {
    double c;
    float c_hi, c_lo;
};
Scale make_scale(double T);

// Kernel-launch tracing (events around each launch when enabled).
void trace_pre(int kernel, hipStream_t s);
void trace_post(hipStream_t s);

// ---- launchers (each enqueues one kernel on `s`) --------------------------------
hipError_t launch_rowstats(const void *tgt, const void *drf, long long rows_t, long long rows_total,
                           int V, const RowGeom &g, sv_dtype dt, const Scale &sc, float *part_R,
                           double *part_s, hipStream_t s);
hipError_t launch_accept(const void *tgt, const void *drf, const int32_t *drafts,
                         const float *ua, const float *us, int B, int K, int V, const RowGeom &g,
                         sv_dtype dt, const Scale &sc, const float *part_R, const double *part_s,
                         double *L2, int32_t *accept_len, int32_t *out_tokens, float *lse_t,
                         float *lse_d, int32_t *status, ResidParam *rp, hipStream_t s);
hipError_t launch_resid_mass(const void *tgt, const void *drf, int B, int V, const RowGeom &g,
                             sv_dtype dt, const Scale &sc, const ResidParam *rp, double *tile_mass,
                             hipStream_t s);
hipError_t launch_resid_select(const void *tgt, const void *drf, int B, int K, int V,
                               const RowGeom &g, sv_dtype dt, const Scale &sc,
                               const ResidParam *rp, double *tile_mass, int32_t *out_tokens,
                               hipStream_t s);
hipError_t launch_argmax(const void *L, long long rows, int V, const RowGeom &g, sv_dtype dt,
                         float *part_v, int32_t *part_i, hipStream_t s);
hipError_t launch_match(const float *part_v, const int32_t *part_i, const int32_t *drafts, int B,
                        int K, int V, const RowGeom &g, int32_t *accept_len, int32_t *out_tokens,
                        int32_t *status, hipStream_t s);
hipError_t launch_tree(const float *part_v, const int32_t *part_i, const int32_t *node_tokens,
                       const int32_t *parents, int B, int N, int V, const RowGeom &g,
                       int32_t *accept_len, int32_t *path_nodes, int32_t *out_tokens,
                       int32_t *status, hipStream_t s);

}  // namespace sv
