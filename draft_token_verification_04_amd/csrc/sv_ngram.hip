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
// tokens at positions c0 + 64 j + lane (j < kNgJ: every load is 64 consecutive
// tokens), plus the 64 tokens before the chunk.  For each j the wave ballots
// the lanes whose token is the anchor; only when one does are the other n - 1
// tokens of each window fetched from neighbouring lanes by shuffles.
//   k_ngram<false>  counts the candidates of each (request, chunk);
//   k_ngram<true>   skips a chunk whose count is zero; otherwise sums the
//                   counts of the earlier chunks of its request and writes its
//                   candidates at that offset, in ascending order; the wave of
//                   chunk 0 writes the request's total and status.
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr int kNgJ = 16;                  // 64-position rows per lane per chunk
constexpr int kNgChunk = kWave * kNgJ;    // positions per wave

template <bool EMIT>
__global__ __launch_bounds__(kBlock) void k_ngram(const int32_t *__restrict__ ctx, long long L,
                                                  const int32_t *__restrict__ lens, int B,
                                                  const int32_t *__restrict__ queries, int n, int nchunks,
                                                  int32_t *__restrict__ counts, int cap,
                                                  int32_t *__restrict__ count,
                                                  int32_t *__restrict__ positions,
                                                  int32_t *__restrict__ status) {
    const int lane = threadIdx.x & (kWave - 1);
    const long long wave = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
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
    const int qreg = lane < n ? queries[static_cast<long long>(b) * n + lane] : 0;
    const int anchor = uniform(__shfl(qreg, n - 1, kWave));
    int tok[kNgJ];
#pragma unroll
    for (int j = 0; j < kNgJ; ++j) {
        const long long p = c0 + j * kWave + lane;
        tok[j] = p < len ? row[p] : 0;
    }
    const long long ph = c0 - kWave + lane;
    const int halo = ph >= 0 ? row[ph] : 0;

    int offset = 0;
    if (EMIT) {
        for (int c = lane; c < chunk; c += kWave) offset += counts[static_cast<long long>(b) * nchunks + c];
        offset = static_cast<int>(wave_sum(static_cast<double>(offset)));
    }
    int found = 0;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
    for (int j = 0; j < kNgJ; ++j) {
        const long long p = c0 + j * kWave + lane;
        bool m = p >= n - 1 && p <= hi && tok[j] == anchor;
        if (ballot(m) == 0) continue;
        const int prev = j > 0 ? tok[j > 0 ? j - 1 : 0] : halo;
        for (int k = 1; k < n; ++k) {
            // token at p - k: this row's lane - k, or the previous row's lane - k + 64
            // (every shuffle runs in all lanes: none sits behind a short-circuit)
            const int here = __shfl(tok[j], (lane - k) & (kWave - 1), kWave);
            const int before = __shfl(prev, (lane - k) & (kWave - 1), kWave);
            const int qk = uniform(__shfl(qreg, n - 1 - k, kWave));
            const int v = lane >= k ? here : before;
            m = m & (v == qk);
        }
        const uint64_t mask = ballot(m);
        if (EMIT && m) {
            const int idx = offset + found + __popcll(mask & below);
            if (idx < cap) positions[static_cast<long long>(b) * cap + idx] = static_cast<int32_t>(p);
        }
        found += __popcll(mask);
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
    trace_select(SV_K_NGRAM_COUNT);
    hipError_t e = launch_kernel(k_ngram<false>, grid, dim3(kBlock), 0, s, ctx, static_cast<long long>(L), lens,
                                 B, queries, n, nchunks, counts, cap, count, positions, status);
    if (e != hipSuccess) return e;
    trace_select(SV_K_NGRAM_EMIT);
    return launch_kernel(k_ngram<true>, grid, dim3(kBlock), 0, s, ctx, static_cast<long long>(L), lens, B,
                         queries, n, nchunks, counts, cap, count, positions, status);
}

}  // namespace sv
