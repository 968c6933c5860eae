// sv_commit.hip -- commit of a verified draft tree's accepted path in the
// target's KV cache.
//
// The AdaPLD page (section 3.3 and Algorithm 1) verifies the whole draft tree
// in one target pass, which leaves one KV row per tree node, and then appends
// the accepted tokens to the context.  Here the rows of the accepted nodes
// (depth 1 first) move into consecutive slots after the context, so the next
// pass sees the committed tokens in order.
//
// One wave per (row group g, request b), four to a workgroup, with no
// synchronisation between waves.  Each wave loads its request's length, bases
// and first path nodes together, checks the path and slots, then copies its d
// rows in chunks of kWave * kCommitVecs 16-byte vectors, in increasing path
// order: it loads the whole chunk, waits for those loads, then stores.  In
// place with commit_base <= tree_base + 1 a write can only land on the source
// row of the same or an earlier path node (node ids grow by at least one per
// level), which this chunk or an earlier one already loaded, so the result is
// that of reading every source first.
#include <algorithm>

#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr int kCommitVecs = 8;  // 16-byte vectors per lane per chunk (v0..v7 below)

// Copies the first `total` vectors of the path rows (row k = path node
// PATH[k], held by lane k in p0 for short paths) in chunks: load the chunk,
// wait for it, store it.  Lanes past the end load the last vector again.
template <bool DEEP>
__device__ __forceinline__ void copy_rows(const uint4 *from, uint4 *into, int total, int row_vecs, int p0,
                                          const int32_t *path, int lane) {
    constexpr int kChunk = kWave * kCommitVecs;
    for (int c0 = 0; c0 < total; c0 += kChunk) {
        uint4 v0, v1, v2, v3, v4, v5, v6, v7;
        auto ld = [&](int t) {
            const int f = min(c0 + t * kWave + lane, total - 1);
            const int k = f / row_vecs;
            const int j = DEEP ? path[k] : __shfl(p0, k, kWave);
            return from[static_cast<long long>(j) * row_vecs + (f - k * row_vecs)];
        };
        v0 = ld(0); v1 = ld(1); v2 = ld(2); v3 = ld(3);
        v4 = ld(4); v5 = ld(5); v6 = ld(6); v7 = ld(7);
        wait_own_stores();  // every load of the chunk has returned before any store
        auto st = [&](int t, const uint4 &v) {
            const int f = c0 + t * kWave + lane;
            if (f < total) {
                const int k = f / row_vecs;
                into[static_cast<long long>(k) * row_vecs + (f - k * row_vecs)] = v;
            }
        };
        st(0, v0); st(1, v1); st(2, v2); st(3, v3);
        st(4, v4); st(5, v5); st(6, v6); st(7, v7);
    }
}

__global__ __launch_bounds__(kBlock) void k_commit(const uint4 *src, uint4 *dst, int G, int B, long long S,
                                                   int row_vecs, const int32_t *__restrict__ tree_base,
                                                   const int32_t *__restrict__ commit_base,
                                                   const int32_t *__restrict__ accept_len,
                                                   const int32_t *__restrict__ path_nodes, int N,
                                                   int in_place, int32_t *__restrict__ status) {
    const int lane = threadIdx.x & (kWave - 1);
    const long long wave = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (wave >= static_cast<long long>(G) * B) return;
    const int b = static_cast<int>(wave % B);
    const int g = static_cast<int>(wave / B);
    const int32_t *path = path_nodes + static_cast<long long>(b) * N;
    const int d = uniform(accept_len[b]);
    const long long tb = uniform(tree_base[b]), cb = uniform(commit_base[b]);
    const int p0 = lane < N ? path[lane] : 0;  // fetched with the scalars above

    // request check (every wave of the request reaches the same verdict)
    int code = 0;
    if (d < 0 || d > N - 1) {
        code = 2;
    } else if (d > 0) {
        bool bad = false;
        int last;
        if (d <= kWave) {
            const int prev = __shfl_up(p0, 1, kWave);
            if (lane < d && (p0 < 1 || p0 >= N || p0 <= (lane == 0 ? 0 : prev))) bad = true;
            last = uniform(__shfl(p0, d - 1, kWave));
        } else {
            for (int k = lane; k < d; k += kWave) {
                const int j = path[k];
                const int prev = k == 0 ? 0 : path[k - 1];
                if (j < 1 || j >= N || j <= prev) bad = true;
            }
            last = uniform(path[d - 1]);
        }
        if (ballot(bad) != 0)
            code = 2;
        else if (tb < 0 || tb + last >= S || cb < 0 || cb + d > S)
            code = 1;
        else if (in_place && cb >= tb + 2 && cb < tb + N)
            code = 3;
    }
    if (g == 0 && lane == 0 && status) status[b] = code;
    if (code != 0 || d == 0) return;

    const long long base = (static_cast<long long>(g) * B + b) * S;  // slot 0 of (g, b)
    const uint4 *from = src + (base + tb) * row_vecs;
    uint4 *into = dst + (base + cb) * row_vecs;
    if (d <= kWave)
        copy_rows<false>(from, into, d * row_vecs, row_vecs, p0, path, lane);
    else
        copy_rows<true>(from, into, d * row_vecs, row_vecs, p0, path, lane);
}

}  // namespace

hipError_t launch_commit(const void *src, void *dst, int G, int B, int S, int row_bytes,
                         const int32_t *tree_base, const int32_t *commit_base,
                         const int32_t *accept_len, const int32_t *path_nodes, int N,
                         int32_t *status, hipStream_t s) {
    const long long waves = static_cast<long long>(G) * B;
    const long long blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    return launch_kernel(k_commit, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s,
                         static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), G, B,
                         static_cast<long long>(S), row_bytes / 16, tree_base, commit_base, accept_len,
                         path_nodes, N, src == dst ? 1 : 0, status);
}

}  // namespace sv
