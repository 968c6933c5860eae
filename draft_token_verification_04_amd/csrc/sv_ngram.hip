// sv_ngram.hip -- AdaPLD's lexical retrieval: every position of a request's
// reuse context where the last n tokens of the current prefix occur.
//
// The AdaPLD page, section 3.2 (lexical retrieval: the newest token is the
// query; candidates are the positions of the reuse context holding it whose
// preceding tokens match the prefix's) and Algorithm 1 (LexicalRetrieval,
// then the main copy path starts after the chosen position, so a candidate
// needs at least one token after it).  Candidate p of request b satisfies
// context[b][p - k] == query[b][n - 1 - k] for k < n, n - 1 <= p <= len - 2.
//
// Two passes over waves of kNgChunk consecutive positions.  A lane holds the
// four tokens at positions c0 + 256 j + 4 lane + e (j < kNgJ rows, e < 4: one
// 16-byte load per row where the row's layout allows), plus the 64 tokens
// before the chunk.  For each (j, e) the wave ballots the lanes whose token is
// the anchor; only when one does are the other n - 1 tokens of each window
// fetched: the token k places before element e of a lane is element
// (e - k) & 3 of the lane floor((e - k) / 4) places back, the same for every
// lane, so one shuffle per k brings it (from the row before when that lane
// lies before lane 0).  The token before the anchor is tested with the anchor
// itself (the lane's own register, or the lane before's last), which leaves
// few windows to fetch.
//   k_ngram<false>  counts the candidates of each (request, chunk);
//   k_ngram<true>   skips a chunk whose count is zero; otherwise sums the
//                   counts of the earlier chunks of its request and writes its
//                   candidates at that offset, in ascending order; the wave of
//                   chunk 0 writes the request's total and status.
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr int kNgRow = kWave * 4;        // positions per row: four per lane
// Rows per chunk (measured on MI355X, µs per call at B=256 and 8K..32K /
// 64K..128K tokens: 2 rows 15.4 / 43.9; 4 rows 15.7 / 33.5; 8 rows 21.3 / 40.3;
// one token per lane, 16 rows of 64: 17.0 / 37.5).
#ifndef SV_NGRAM_ROWS
#define SV_NGRAM_ROWS 4
#endif
constexpr int kNgJ = SV_NGRAM_ROWS;
constexpr int kNgChunk = kNgRow * kNgJ;  // positions per wave

// Element e of four registers, e uniform.
__device__ __forceinline__ int pick4(const int (&t)[4], int e) {
    return e == 0 ? t[0] : (e == 1 ? t[1] : (e == 2 ? t[2] : t[3]));
}

// VEC: the context's rows are 16-byte aligned (L % 4 == 0 and an aligned
// base), so a row's four tokens per lane come in one load.
template <bool EMIT, bool VEC>
__global__ __launch_bounds__(kBlock) void k_ngram(const int32_t *__restrict__ ctx, long long L,
                                                  const int32_t *__restrict__ lens, int B,
                                                  const int32_t *__restrict__ queries, int n, int nchunks,
                                                  int32_t *__restrict__ counts, int cap,
                                                  int32_t *__restrict__ count,
                                                  int32_t *__restrict__ positions,
                                                  int32_t *__restrict__ status) {
    const int lane = threadIdx.x & (kWave - 1);
    // the wave index as a scalar: the request's length then comes in through
    // the scalar cache, not behind other waves' streaming loads
    const long long wave =
        static_cast<long long>(blockIdx.x) * kWavesPerBlock + uniform(static_cast<int>(threadIdx.x >> 6));
    if (wave >= static_cast<long long>(B) * nchunks) return;
    const int b = static_cast<int>(wave / nchunks);
    const int chunk = static_cast<int>(wave - static_cast<long long>(b) * nchunks);
    const int len = uniform(lens[b]);
    const bool bad = len < 0 || len > L;
    if (!EMIT) {
        // the padding of the positions array comes first (the emit pass overwrites it)
        if (chunk == 0)
            for (int i = lane; i < cap; i += kWave) positions[static_cast<long long>(b) * cap + i] = -1;
    } else if (chunk == 0) {
        int tot = 0;
        if (!bad)
            for (int c = lane; c < nchunks; c += kWave) tot += counts[static_cast<long long>(b) * nchunks + c];
        tot = static_cast<int>(wave_sum(static_cast<double>(tot)));
        if (lane == 0) {
            count[b] = bad ? 0 : tot;
            if (status) status[b] = bad ? 1 : 0;
        }
    }
    const long long c0 = static_cast<long long>(chunk) * kNgChunk;
    const long long hi = static_cast<long long>(len) - 2;  // last position with a continuation
    if (bad || c0 > hi || hi < n - 1) {
        if (!EMIT && lane == 0) counts[static_cast<long long>(b) * nchunks + chunk] = 0;
        return;
    }
    // a chunk without candidates has nothing to emit (most chunks: candidates are rare)
    if (EMIT && uniform(counts[static_cast<long long>(b) * nchunks + chunk]) == 0) return;
    const int32_t *row = ctx + static_cast<long long>(b) * L;
    // only tokens before position len - 1 can belong to a candidate's window
    int tok[kNgJ][4];
#pragma unroll
    for (int j = 0; j < kNgJ; ++j) {
        const long long p0 = c0 + j * kNgRow + 4 * lane;
        if (VEC && p0 + 3 < len) {
            // the counting pass streams the context once (non-temporal); the
            // emit pass re-reads only chunks with candidates
            const u32x4 v = EMIT ? *reinterpret_cast<const u32x4 *>(row + p0)
                                 : __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + p0));
            tok[j][0] = static_cast<int>(v.x);
            tok[j][1] = static_cast<int>(v.y);
            tok[j][2] = static_cast<int>(v.z);
            tok[j][3] = static_cast<int>(v.w);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) tok[j][e] = p0 + e < len ? row[p0 + e] : 0;
        }
    }
    // the 64 tokens before the chunk, in the last 16 lanes (a window reaches
    // back at most 63 tokens)
    int halo[4];
    {
        const long long p0 = c0 - kNgRow + 4 * lane;
#pragma unroll
        for (int e = 0; e < 4; ++e) halo[e] = lane >= kWave - 16 && p0 + e >= 0 ? row[p0 + e] : 0;
    }
    // the query after the context loads, so they do not wait for it
    const int qreg = lane < n ? queries[static_cast<long long>(b) * n + lane] : 0;
    const int anchor = uniform(__shfl(qreg, n - 1, kWave));

    int offset = 0;
    if (EMIT) {
        for (int c = lane; c < chunk; c += kWave) offset += counts[static_cast<long long>(b) * nchunks + c];
        offset = static_cast<int>(wave_sum(static_cast<double>(offset)));
    }
    int found = 0;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
    const int q1 = n >= 2 ? uniform(__shfl(qreg, n - 2, kWave)) : 0;
#pragma unroll
    for (int j = 0; j < kNgJ; ++j) {
        const int(&prev)[4] = j > 0 ? tok[j > 0 ? j - 1 : 0] : halo;
        // the token before each of the lane's four: the lane's own, or the
        // last of the lane before (for lane 0, of the row before)
        const int left = __shfl(tok[j][3], (lane - 1) & (kWave - 1), kWave);
        const int left0 = __shfl(prev[3], kWave - 1, kWave);
        const int t1[4] = {lane > 0 ? left : left0, tok[j][0], tok[j][1], tok[j][2]};
        bool m[4];
        uint64_t M[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const long long p = c0 + j * kNgRow + 4 * lane + e;
            // the last two tokens of the window first: most anchors fail there
            m[e] = p >= n - 1 && p <= hi && tok[j][e] == anchor && (n < 2 || t1[e] == q1);
            M[e] = ballot(m[e]);
            if (M[e] == 0 || n < 3) continue;
            for (int k = 2; k < n; ++k) {
                // token at p - k: element (e - k) & 3 of lane + d, d = floor((e - k) / 4),
                // in this row, or in the row before when lane + d < 0 (every shuffle
                // runs in all lanes: none sits behind a short-circuit)
                const int d = (e - k) >> 2;
                const int es = (e - k) & 3;
                const int src = (lane + d) & (kWave - 1);
                const int here = __shfl(pick4(tok[j], es), src, kWave);
                const int before = __shfl(pick4(prev, es), src, kWave);
                const int qk = uniform(__shfl(qreg, n - 1 - k, kWave));
                const int v = lane + d >= 0 ? here : before;
                m[e] = m[e] & (v == qk);
            }
            M[e] = ballot(m[e]);
        }
        const int row_hits = __popcll(M[0]) + __popcll(M[1]) + __popcll(M[2]) + __popcll(M[3]);
        if (EMIT && row_hits > 0) {
            // ascending order within the row: by lane, then by element
            int rank = offset + found + __popcll(M[0] & below) + __popcll(M[1] & below) +
                       __popcll(M[2] & below) + __popcll(M[3] & below);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (m[e]) {
                    if (rank < cap)
                        positions[static_cast<long long>(b) * cap + rank] =
                            static_cast<int32_t>(c0 + j * kNgRow + 4 * lane + e);
                    ++rank;
                }
            }
        }
        found += row_hits;
    }
    if (!EMIT && lane == 0) counts[static_cast<long long>(b) * nchunks + chunk] = found;
}

}  // namespace

int ngram_chunks(int L) { return (L + kNgChunk - 1) / kNgChunk; }

hipError_t launch_ngram(const int32_t *ctx, int B, int L, const int32_t *lens, const int32_t *queries,
                        int n, int cap, int32_t *counts, int32_t *count, int32_t *positions,
                        int32_t *status, hipStream_t s) {
    const int nchunks = ngram_chunks(L);
    const long long waves = static_cast<long long>(B) * nchunks;
    const dim3 grid(static_cast<unsigned>((waves + kWavesPerBlock - 1) / kWavesPerBlock));
    const bool vec = (reinterpret_cast<uintptr_t>(ctx) & 15u) == 0 && (L & 3) == 0;
    trace_select(SV_K_NGRAM_COUNT);
    hipError_t e = launch_kernel(vec ? k_ngram<false, true> : k_ngram<false, false>, grid, dim3(kBlock), 0, s,
                                 ctx, static_cast<long long>(L), lens, B, queries, n, nchunks, counts, cap, count,
                                 positions, status);
    if (e != hipSuccess) return e;
    trace_select(SV_K_NGRAM_EMIT);
    return launch_kernel(vec ? k_ngram<true, true> : k_ngram<true, false>, grid, dim3(kBlock), 0, s, ctx,
                         static_cast<long long>(L), lens, B, queries, n, nchunks, counts, cap, count, positions,
                         status);
}

}  // namespace sv
