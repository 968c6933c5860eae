// sv_greedy.hip -- greedy verification of draft chains and draft trees.
//
// Chains follow the greedy rule on the speculative-decoding tutorial page,
// section "为什么“猜错再改”不会偏离目标分布": a draft is accepted while it equals
// the target's argmax, and the target's token is emitted at the first mismatch
// (or after the last draft, as the bonus).  Trees follow the AdaPLD page,
// section 3.3 and Algorithm 1 (BuildDraftTree / VerifyAndAccept): node j is
// accepted when its parent is and its token is the argmax of its parent's row;
// the deepest accepted node (lowest index among equals) ends the accepted path,
// and the argmax of its own row is the bonus token.
//
// Kernels:
//   k_argmax  one streaming pass over the target rows; each wave reduces a
//             segment to (max value, lowest index of that value), packed in one
//             64-bit key whose maximum is the row argmax with ties to the
//             lowest index.
//   k_match   one workgroup per request: stages the row keys in LDS, one wave
//             per row reduces them, then a ballot finds the first mismatch.
//   k_tree    one workgroup per request: the same key merge per node, the
//             parent-array check in parallel, acceptance and depth of every
//             node by pointer jumping (log2 N rounds), the deepest accepted
//             node by an LDS max, then the path write-out.
//   k_chain_prep, k_skip_argmax  chains with K <= 31: a small launch clears
//             each request's words and finds, from a sample of each draft's
//             row, the first draft that cannot be the argmax; then one launch
//             that does not read the rows after each request's first mismatch
//             (the protocol is described with SkipCtl); the decision of
//             position p is the row argmax compared with draft p.
//   k_tree_prep, k_skip_tree  trees with N <= 64: a small launch clears the
//             control words, rejects the nodes a sample of their parent's row
//             rules out and ranks the rest by depth, then one launch reads
//             the node rows level by level, skipping the rows of nodes
//             already known rejected (described with TreeCtl).
#include <limits.h>

#include <algorithm>

#include "sv_device.hpp"
#include "sv_internal.hpp"
#include "sv_skip.hpp"

namespace sv {
namespace {

template <typename E, bool ALIGNED, int U>
__global__ __launch_bounds__(kBlock) void k_argmax(const typename E::storage *__restrict__ L,
                                                   long long nwaves, int V, int nvec, int segs,
                                                   uint64_t *__restrict__ part_k) {
    constexpr int P = E::kPerVec;
    const int lane = threadIdx.x & (kWave - 1);
    const long long wave = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (wave >= nwaves) return;
    const long long row = wave / segs;
    const int seg = static_cast<int>(wave - row * segs);
    const typename E::storage *base = L + row * static_cast<long long>(V);
    const int v0 = static_cast<int>((static_cast<long long>(seg) * nvec) / segs);
    const int v1 = static_cast<int>((static_cast<long long>(seg + 1) * nvec) / segs);

    Staged<E, ALIGNED> st[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int j = v0 + k * kWave + lane;
        if (j < v1)
            st[k].load(base, V, j);
        else
            st[k].set_neg_inf();
    }
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int k = 0; k < U; ++k) {
        float x[P];
        st[k].get(x);
#pragma unroll
        for (int e = 0; e < P; ++e) m = fmaxf(m, x[e]);
    }
    m = wave_max(m);
    // lowest element index holding the maximum (floats compare equal for -0/+0)
    int cand = INT_MAX;
#pragma unroll
    for (int k = U - 1; k >= 0; --k) {
        const int j = v0 + k * kWave + lane;
        float x[P];
        st[k].get(x);
#pragma unroll
        for (int e = P - 1; e >= 0; --e)
            if (j < v1 && x[e] == m) cand = j * P + e;
    }
    cand = wave_min(cand);
    if (lane == 0) part_k[wave] = argmax_key(m, cand);
}

// Argmax of `nrows` consecutive rows whose segment keys start at `keys`
// (segs keys per row), written to out[0..nrows).  The keys of up to
// `lds_rows` rows at a time are first copied into LDS with every load in
// flight; then each wave reduces whole rows.  lds_rows = 0 reads global memory
// directly (rows with too many segments to stage).  Each thread loads
// kKeyUnroll keys before it uses any of them: a row of the fused projection has
// ~1200 keys, and one memory latency per key would dominate.
constexpr int kKeyUnroll = 8;
__device__ __forceinline__ void merge_rows(const uint64_t *__restrict__ keys, int nrows, int segs,
                                           int lds_rows, uint64_t *stage, int *out) {
    constexpr int U = kKeyUnroll;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & (kWave - 1);
    const int nw = blockDim.x >> 6;
    const int chunk = lds_rows > 0 ? lds_rows : nrows;
    for (int r0 = 0; r0 < nrows; r0 += chunk) {
        const int nr = min(chunk, nrows - r0);
        const uint64_t *src = keys + static_cast<long long>(r0) * segs;
        if (lds_rows > 0) {
            const int n = nr * segs;
            for (int i0 = tid; i0 < n; i0 += U * static_cast<int>(blockDim.x)) {
                uint64_t v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = i0 + u * static_cast<int>(blockDim.x);
                    v[u] = i < n ? src[i] : 0;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = i0 + u * static_cast<int>(blockDim.x);
                    if (i < n) stage[i] = v[u];
                }
            }
            __syncthreads();
            src = stage;
        }
        for (int rr = wid; rr < nr; rr += nw) {
            uint64_t mk = 0;
            for (int s0 = lane; s0 < segs; s0 += U * kWave) {
                uint64_t v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = s0 + u * kWave < segs ? src[rr * segs + s0 + u * kWave] : 0;
#pragma unroll
                for (int u = 0; u < U; ++u) mk = v[u] > mk ? v[u] : mk;
            }
            mk = wave_max_u64(mk);
            if (lane == 0) out[r0 + rr] = argmax_key_index(mk);
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kBlock) void k_match(const uint64_t *__restrict__ part_k, int segs,
                                                  int lds_rows, const int32_t *__restrict__ drafts,
                                                  int B, int K, int V,
                                                  int32_t *__restrict__ accept_len,
                                                  int32_t *__restrict__ out_tokens,
                                                  int32_t *__restrict__ status) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint64_t *stage = reinterpret_cast<uint64_t *>(smem);
    int *s_a = reinterpret_cast<int *>(stage + static_cast<size_t>(lds_rows) * segs);
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int32_t *xb = drafts + static_cast<long long>(b) * K;
    const int x0 = tid < K ? xb[tid] : -1;  // first 64 drafts, fetched while the keys are merged
    merge_rows(part_k + static_cast<long long>(b) * (K + 1) * segs, K + 1, segs, lds_rows, stage, s_a);
    if (tid >= kWave) return;
    int n = K;
    bool bad = false;
    for (int i0 = 0; i0 < K; i0 += kWave) {
        const int i = i0 + lane;
        bool stop = false;
        if (i < K) {
            const int x = i0 == 0 ? x0 : xb[i];
            if (x < 0 || x >= V) bad = true;
            stop = x != s_a[i];
        }
        const uint64_t mk = ballot(stop);
        if (mk != 0 && n == K) n = i0 + first_lane(mk);
    }
    const bool any_bad = ballot(bad) != 0;
    int32_t *tok = out_tokens + static_cast<long long>(b) * (K + 1);
    for (int i = lane; i <= K; i += kWave)
        tok[i] = i < n ? (i < kWave ? x0 : xb[i]) : (i == n ? s_a[n] : -1);
    if (lane == 0) {
        accept_len[b] = n;
        if (status) status[b] = any_bad ? 1 : 0;
    }
}

// Nodes per thread in the tree kernel (SV_MAX_TREE_NODES / kBlock).
constexpr int kTreeNodesPerThread = (SV_MAX_TREE_NODES + kBlock - 1) / kBlock;

__global__ __launch_bounds__(kBlock) void k_tree(const uint64_t *__restrict__ part_k, int segs,
                                                 int lds_rows,
                                                 const int32_t *__restrict__ node_tokens,
                                                 const int32_t *__restrict__ parents, int B, int N,
                                                 int V, int32_t *__restrict__ accept_len,
                                                 int32_t *__restrict__ path_nodes,
                                                 int32_t *__restrict__ out_tokens,
                                                 int32_t *__restrict__ status) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint64_t *stage = reinterpret_cast<uint64_t *>(smem);
    int *s_a = reinterpret_cast<int *>(stage + static_cast<size_t>(lds_rows) * segs);  // argmax per node
    int *s_par = s_a + N;     // parents
    int *s_tok = s_par + N;   // node tokens
    int *s_ok = s_tok + N;    // accepted along the whole path to the root
    int *s_dep = s_ok + N;    // depth
    int *s_anc = s_dep + N;   // pointer-jumping ancestor, then the chosen path
    __shared__ int s_bad, s_oor;
    __shared__ unsigned s_key;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_bad = 0;
        s_oor = 0;
        s_key = 0;
    }
    const long long base = static_cast<long long>(b) * N;
    for (int j = tid; j < N; j += kBlock) {
        s_par[j] = parents[base + j];
        s_tok[j] = node_tokens[base + j];
    }
    merge_rows(part_k + base * segs, N, segs, lds_rows, stage, s_a);  // ends with a barrier
    for (int j = tid; j < N; j += kBlock) {
        const int p = s_par[j];
        if (j == 0 ? p != -1 : (p < 0 || p >= j)) atomicOr(&s_bad, 1);
        if (j > 0 && (s_tok[j] < 0 || s_tok[j] >= V)) atomicOr(&s_oor, 1);
    }
    __syncthreads();
    if (s_bad) {
        for (int k = tid; k < N; k += kBlock) {
            path_nodes[base + k] = -1;
            out_tokens[base + k] = -1;
        }
        if (tid == 0) {
            accept_len[b] = -1;
            if (status) status[b] = 2;
        }
        return;
    }
    // Pointer jumping: after round r every node has folded in the acceptance
    // and depth of its 2^r nearest ancestors; the root is the fixed point.
    for (int j = tid; j < N; j += kBlock) {
        const int p = s_par[j];
        s_anc[j] = j == 0 ? 0 : p;
        s_ok[j] = j == 0 ? 1 : (s_tok[j] == s_a[p] ? 1 : 0);
        s_dep[j] = j == 0 ? 0 : 1;
    }
    __syncthreads();
    for (int span = 1; span < N; span <<= 1) {
        int ok2[kTreeNodesPerThread], d2[kTreeNodesPerThread], a2[kTreeNodesPerThread];
#pragma unroll
        for (int t = 0; t < kTreeNodesPerThread; ++t) {
            const int j = tid + t * kBlock;
            if (j < N) {
                const int a = s_anc[j];
                ok2[t] = s_ok[a];
                d2[t] = s_dep[a];
                a2[t] = s_anc[a];
            }
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kTreeNodesPerThread; ++t) {
            const int j = tid + t * kBlock;
            if (j < N) {
                s_ok[j] &= ok2[t];
                s_dep[j] += d2[t];
                s_anc[j] = a2[t];
            }
        }
        __syncthreads();
    }
    // deepest accepted node, lowest index among equals (the root always qualifies)
    for (int j = tid; j < N; j += kBlock)
        if (s_ok[j]) atomicMax(&s_key, (static_cast<unsigned>(s_dep[j]) << 16) | (0xffffu - static_cast<unsigned>(j)));
    __syncthreads();
    const int best = static_cast<int>(0xffffu - (s_key & 0xffffu));
    const int d = static_cast<int>(s_key >> 16);
    if (tid == 0)
        for (int j = best, k = d - 1; j != 0; j = s_par[j], --k) s_anc[k] = j;  // the path, depth 1 first
    __syncthreads();
    for (int k = tid; k < N; k += kBlock) {
        path_nodes[base + k] = k < d ? s_anc[k] : -1;
        out_tokens[base + k] = k < d ? s_tok[s_anc[k]] : (k == d ? s_a[best] : -1);
    }
    if (tid == 0) {
        accept_len[b] = d;
        if (status) status[b] = s_oor ? 1 : 0;
    }
}

// Argmax key of vectors [v0, v1) of one row, read in CH chunks of U vectors
// per lane, each chunk loaded while the previous one is scanned.  A lane visits
// its vectors in increasing index and keeps the first whose maximum is strictly
// greater than every earlier one (-0 and +0 compare equal), together with that
// vector's raw contents; the lowest element of the kept vector equal to the
// maximum is then the lane's argmax.  The wave's largest key is the segment
// maximum with the lowest index among equals.  A lane whose elements are all
// -inf keeps its first element, as the full-read pass does.
template <typename E, bool ALIGNED, int U, int CH>
__device__ __forceinline__ uint64_t segment_argmax_chunked(const typename E::storage *__restrict__ base,
                                                           int V, int v0, int v1, int lane) {
    constexpr int P = E::kPerVec;
    Staged<E, ALIGNED> a[U], b[U], keep;
    keep.set_neg_inf();
    float best = -__builtin_huge_valf();
    int bk = 0;  // kept vector, counted in steps of kWave vectors from v0 + lane
    auto load = [&](Staged<E, ALIGNED>(&st)[U], int c0) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int j = c0 + k * kWave + lane;
            if (j < v1)
                st[k].load(base, V, j);
            else
                st[k].set_neg_inf();
        }
    };
    auto scan = [&](const Staged<E, ALIGNED>(&st)[U], int ch) {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float x[P];
            st[k].get(x);
            float vm = x[0];
#pragma unroll
            for (int e = 1; e < P; ++e) vm = fmaxf(vm, x[e]);
            if (vm > best) {
                best = vm;
                bk = ch * U + k;
                keep = st[k];
            }
        }
    };
    constexpr int step = kWave * U;
    load(a, v0);
#pragma unroll
    for (int ch = 0; ch < CH; ch += 2) {
        if (ch + 1 < CH) load(b, v0 + (ch + 1) * step);
        scan(a, ch);
        if (ch + 2 < CH) load(a, v0 + (ch + 2) * step);
        if (ch + 1 < CH) scan(b, ch + 1);
    }
    float x[P];
    keep.get(x);
    int e0 = P - 1;
#pragma unroll
    for (int e = P - 2; e >= 0; --e)
        if (x[e] == best) e0 = e;
    const int idx = v0 + lane < v1 ? (v0 + lane + bk * kWave) * P + e0 : INT_MAX;
    return wave_max_u64(argmax_key(best, idx));
}

template <typename E, bool ALIGNED, int U>
__global__ __launch_bounds__(kBlock) void k_skip_argmax(const typename E::storage *__restrict__ L,
                                                        const int32_t *__restrict__ drafts, int B, int K,
                                                        int V, int nvec, int segs, uint64_t *part_k,
                                                        int32_t *amax, SkipCtl ctl, int early, int rot,
                                                        int32_t *__restrict__ accept_len,
                                                        int32_t *__restrict__ out_tokens,
                                                        int32_t *__restrict__ status) {
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned wave = skip_wave_index();
    const unsigned per_pos = static_cast<unsigned>(B) * static_cast<unsigned>(segs);
    if (wave >= per_pos * static_cast<unsigned>(K + 1)) return;
    const int p = static_cast<int>(wave / per_pos);
    const unsigned rem = wave - static_cast<unsigned>(p) * per_pos;
    const unsigned slot = rem / static_cast<unsigned>(segs);
    const int sg = static_cast<int>(rem - slot * static_cast<unsigned>(segs));
    const int b = skip_request(slot, p, B, rot);
    // position 0's rows are always needed: no test, no wait before their loads.
    // Rows past the request's sampled rejection are dead from the start (a
    // plain word the preparing launch wrote); the others are tested against
    // the decisions recorded so far
    if (p > 0) {
        const unsigned lim = uniform(ctl.lim[b]);
        const bool dead = early ? skip_row_dead(ctl, b, p) : uniform(shared_load(&ctl.finished[b])) != 0;
        if (static_cast<unsigned>(p) > lim || dead) return;
    }

    const long long row = static_cast<long long>(b) * (K + 1) + p;
    int v0, v1;
    skip_segment(sg, nvec, segs, v0, v1);
    // the row's last segment decides position p: the request's drafts (one
    // per lane, K <= 31) are fetched before the segment's loads and read only
    // at the decision, and by the finisher
    const int32_t *xb = drafts + static_cast<long long>(b) * K;
    const int xl = sg == segs - 1 && lane < K ? xb[lane] : 0;
    const uint64_t key = segment_argmax_chunked<E, ALIGNED, U, kGSkipChunks>(L + row * V, V, v0, v1, lane);
    // Every wave leaves its segment's key (never 0; the keys start at 0) and
    // goes; the wave of the row's last segment, dispatched after all the
    // others, collects them and decides.  A key it waits for is either on its
    // way or was never written because its wave found the request already
    // settled, which the same test then tells this wave too.
    if (sg != segs - 1) {
        if (lane == 0) shared_store(&part_k[row * segs + sg], key);
        return;
    }
    uint64_t mk = key;
    bool complete = false;
    for (int t = 0; t < kSkipPollCap; ++t) {
        uint64_t m = 0;
        bool missing = false;
        for (int s = lane; s < segs - 1; s += kWave) {
            const uint64_t k = shared_load(&part_k[row * segs + s]);
            missing |= k == 0;
            m = k > m ? k : m;
        }
        if (ballot(missing) == 0) {
            mk = wave_max_u64(m > mk ? m : mk);
            complete = true;
            break;
        }
        if (early ? skip_row_dead(ctl, b, p) : uniform(shared_load(&ctl.finished[b])) != 0) return;
        __builtin_amdgcn_s_sleep(2);
    }
    if (!complete) return;  // never decide on part of a row
    const int a = uniform(argmax_key_index(mk));
    uint64_t bits = 1ull << p;
    if (p < K && uniform(__shfl(xl, p, kWave)) != a) bits |= 1ull << (32 + p);
    // amax holds each decided row's argmax plus one (0: not yet known); the
    // store need not land before the decision, the finisher polls for it
    uint64_t old = 0;
    if (lane == 0) {
        shared_store(&amax[row], a + 1);
        old = __hip_atomic_fetch_or(&ctl.mask[b], bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    old = uniform(static_cast<uint64_t>(__shfl(static_cast<long long>(old), 0, kWave)));
    if (skip_prefix(old, K) >= 0) return;  // the request was complete already
    const int n = skip_prefix(old | bits, K);
    if (n < 0) return;
    int an = a;
    if (n != p) {
        int v = 0;
        if (lane == 0) {
            int32_t *w = &amax[static_cast<long long>(b) * (K + 1) + n];
            for (int t = 0; t < kSkipPollCap && (v = shared_load(w)) == 0; ++t) __builtin_amdgcn_s_sleep(1);
        }
        an = uniform(__shfl(v, 0, kWave)) - 1;
    }
    bool bad = false;
    int32_t *tok = out_tokens + static_cast<long long>(b) * (K + 1);
    for (int i = lane; i <= K; i += kWave) {  // K <= 31: lane i holds draft i
        const int x = i < K ? xl : 0;
        if (i < K && (x < 0 || x >= V)) bad = true;
        tok[i] = i < n ? x : (i == n ? an : -1);
    }
    const bool any_bad = ballot(bad) != 0;
    if (lane == 0) {
        accept_len[b] = n;
        if (status) status[b] = any_bad ? 1 : 0;
    }
    skip_finished(ctl, b, lane);
}

// Per request of a greedy chain (one workgroup): clear the request's control
// words, segment keys and argmax words, and sample the rows of its drafts.
// The sample is a row's first 64 vectors (512 bf16 logits); when its largest
// logit is above the logit of the row's draft, that draft is not the row's
// argmax and is rejected.  The first such position r is recorded before any
// row is streamed as the limit past which no row of the request is read; row
// r itself is read, and its decision (a mismatch) records the rejection and
// supplies the emitted argmax, so the decisions run as without the sample.
// A draft outside the vocabulary counts as rejected, as in the decision.  With drafts that are either the
// argmax or an unrelated token this finds almost every mismatch at once (an
// unrelated token tops a 512-logit sample about once in 500); the others are
// left to the decisions.
constexpr int kChainPrepRows = kSkipMaxK / kWavesPerBlock + 1;  // sampled rows per wave
template <typename E, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void k_chain_prep(const typename E::storage *__restrict__ L,
                                                       const int32_t *__restrict__ drafts, int B, int K, int V,
                                                       int nvec, int segs, SkipCtl ctl,
                                                       uint64_t *__restrict__ part_k, int32_t *__restrict__ amax) {
    constexpr int R = kChainPrepRows;
    constexpr int kPad = kWave + 4;
    __shared__ __align__(16) float s_part[(kSkipMaxK + 1) * kPad];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x >> 6;
    const int b = blockIdx.x;
    if (b >= B) return;
    const long long r0 = static_cast<long long>(b) * (K + 1);
    int d = -1;
    if (wid == 0 && lane < K) d = drafts[static_cast<long long>(b) * K + lane];
    const int sv = min(nvec, kWave);
    Staged<E, ALIGNED> st[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int p = wid + k * kWavesPerBlock;
        if (p < K && lane < sv)
            st[k].load(L + (r0 + p) * static_cast<long long>(V), V, lane);
        else
            st[k].set_neg_inf();
    }
    const bool dv = wid == 0 && lane < K && d >= 0 && d < V;
    unsigned xb = 0;
    if (dv) xb = storage_bits(L[(r0 + lane) * static_cast<long long>(V) + d]);
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int p = wid + k * kWavesPerBlock;
        if (p < K) {  // uniform
            float x[E::kPerVec];
            st[k].get(x);
            float m = x[0];
#pragma unroll
            for (int e = 1; e < E::kPerVec; ++e) m = fmaxf(m, x[e]);
            s_part[p * kPad + lane] = m;
        }
    }
    // the words every wave of the request's rows reads start at 0
    for (int i = threadIdx.x; i < (K + 1) * segs; i += kBlock) part_k[r0 * segs + i] = 0;
    if (threadIdx.x <= K) amax[r0 + threadIdx.x] = 0;
    __syncthreads();
    if (wid != 0) return;
    float smax = -__builtin_huge_valf();
    if (lane < K) {
        const float4 *r4 = reinterpret_cast<const float4 *>(s_part + lane * kPad);
#pragma unroll
        for (int i = 0; i < kWave / 4; ++i) {
            const float4 v = r4[i];
            smax = fmaxf(smax, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
        }
    }
    const uint64_t rej = ballot(lane < K && (!dv || smax > from_bits<E>(xb)));
    const int r = rej ? first_lane(rej) : K;
    if (lane == 0) {
        ctl.mask[b] = 0ull;
        ctl.finished[b] = 0u;
        ctl.lim[b] = static_cast<unsigned>(r);
    }
}

// ---- trees: rows of rejected nodes are not read (N <= 64) ------------------------
//
// A node's row is needed only when the node is accepted: its argmax decides its
// children and, for the chosen node, the bonus.  A first small launch
// (k_tree_prep, one workgroup per request) clears the control words, rejects
// the nodes that a sample of their parent's row already rules out, and ranks
// the request's live nodes by (depth, index) ahead of the rejected ones: slot
// i of the request holds the node of rank i, and the slots from the live count
// on are never read.  The main launch runs over every (slot i, request b, segment) in
// slot order, so every node of depth d is read before any of depth d + 1 and
// the decisions about a level have usually landed before the next level's
// waves start (in plain index order, a deep chain listed early would be read
// before its first node is decided).  A wave skips its segment when the node of
// its slot is already known rejected.  The last wave of a row takes its
// argmax a_j, marks the row done, and rejects every child
// whose token differs from a_j together with the descendants of every rejected
// node (parents, tokens and states of the request's nodes held one per lane,
// the rejection closed over the tree by ballots).  Each node is resolved once -
// row done or rejected, whichever is first - and counted; the wave whose count
// completes the request's N nodes walks the tree (every node that is not
// rejected has its row's argmax) and writes the outputs, exactly as the
// full-read walk would.  Nothing waits.

constexpr unsigned kRowDone = 1u, kRejected = 2u;
constexpr int kTreeSkipMaxN = kWave;

struct TreeCtl {
    unsigned *state;     // [B*N] kRowDone | kRejected of the node in each slot
    unsigned *resolved;  // [B] nodes resolved
    int32_t *order;      // [B*N] node of each slot (ascending depth, then index)
    int32_t *rank;       // [B*N] slot of each node
    unsigned *nlive;     // [B] nodes not rejected by the row samples (slots 0 .. nlive-1)
};

// Per request (one workgroup): sample each node's row, clear the request's
// control words and rank its nodes.  The sample is the row's first 64 vectors
// (512 bf16 logits).  A child whose token's logit in its parent's row is below
// the largest logit of that row's sample cannot be the row's argmax, so it is
// rejected before any row is streamed, with every node under it.  With drafts
// that are either the argmax or an unrelated token this settles almost every
// rejection at once (an unrelated token tops a 512-logit sample about once in
// 500); the rest are left to the decisions.  Depths come from pointer jumping
// over the lanes; a parent outside [0, j) counts as the root for the depth and
// passes no rejection down (the walk flags such a request).  The live nodes
// take slots 0 .. nlive-1 by (depth, index), the rejected ones the slots after
// them, so the slots are always a permutation of the nodes.
template <typename E, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void k_tree_prep(const typename E::storage *__restrict__ L,
                                                      const int32_t *__restrict__ par,
                                                      const int32_t *__restrict__ tok, int B, int N, int V,
                                                      int nvec, TreeCtl ctl, uint64_t *__restrict__ part_k,
                                                      int segs) {
    constexpr int P = E::kPerVec;
    constexpr int R = kTreeSkipMaxN / kWavesPerBlock;  // rows sampled per wave
    constexpr int kPad = kWave + 4;                    // 16-byte aligned rows of partial maxima
    __shared__ __align__(16) float s_part[kTreeSkipMaxN * kPad];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x >> 6;
    const int b = blockIdx.x;
    if (b >= B) return;
    const long long base = static_cast<long long>(b) * N;
    const bool in = lane < N;
    // wave 0 fetches the request's parents and tokens, then each node's token
    // logit in its parent's row, while every wave samples its rows
    int p = 0, t = 0;
    if (wid == 0 && in) {
        p = par[base + lane];
        t = tok[base + lane];
    }
    const int sv = min(nvec, kWave);
    Staged<E, ALIGNED> st[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int j = wid + k * kWavesPerBlock;
        if (j < N && lane < sv)
            st[k].load(L + (base + j) * static_cast<long long>(V), V, lane);
        else
            st[k].set_neg_inf();
    }
    const bool pv = wid == 0 && in && lane > 0 && p >= 0 && p < N;
    const bool tv = t >= 0 && t < V;
    unsigned xb = 0;
    if (pv && tv) xb = storage_bits(L[(base + p) * static_cast<long long>(V) + t]);
    // depths (wave 0), while the samples and the token logits are in flight
    const bool topo = lane > 0 && p >= 0 && p < lane;  // a parent listed before its child
    int dep = 0;
    if (wid == 0) {
        int anc = (lane == 0 || !in || !topo) ? 0 : p;
        dep = (lane == 0 || !in) ? 0 : 1;
        for (int span = 1; span < N; span <<= 1) {
            const int d2 = __shfl(dep, anc, kWave);
            const int a2 = __shfl(anc, anc, kWave);
            dep += d2;
            anc = a2;
        }
    }
    // each lane's largest sampled logit of each row, reduced per row below
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int j = wid + k * kWavesPerBlock;
        if (j < N) {  // uniform
            float x[P];
            st[k].get(x);
            float m = x[0];
#pragma unroll
            for (int e = 1; e < P; ++e) m = fmaxf(m, x[e]);
            s_part[j * kPad + lane] = m;
        }
    }
    {  // the segment keys of the request's rows start at 0
        uint64_t *pk = part_k + base * segs;
        for (int i = threadIdx.x; i < N * segs; i += kBlock) pk[i] = 0;
    }
    __syncthreads();
    if (wid != 0) return;

    float smax = -__builtin_huge_valf();  // lane j: the largest sampled logit of row j
    if (in) {
        const float4 *r4 = reinterpret_cast<const float4 *>(s_part + lane * kPad);
#pragma unroll
        for (int i = 0; i < kWave / 4; ++i) {
            const float4 v = r4[i];
            smax = fmaxf(smax, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
        }
    }
    const float sp = __shfl(smax, pv ? p : 0, kWave);
    // a token outside the vocabulary can never be the argmax
    uint64_t dead = ballot(pv && (!tv || sp > from_bits<E>(xb)));
    for (int it = 0; it < N; ++it) {  // close over the tree, as the decisions do
        const uint64_t d2 = dead | ballot(in && topo && ((dead >> p) & 1ull));
        if (d2 == dead) break;  // uniform
        dead = d2;
    }
    const bool is_dead = in && ((dead >> lane) & 1ull);
    const unsigned key = in ? ((is_dead ? 1u << 16 : 0u) | (static_cast<unsigned>(dep) << 8) | static_cast<unsigned>(lane))
                            : 0xffffffffu;
    int rk = 0;
    for (int o = 0; o < N; ++o)
        rk += static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(key), o)) < key;
    const int ndead = __popcll(dead);
    if (in) {
        ctl.order[base + rk] = lane;
        ctl.rank[base + lane] = rk;
        ctl.state[base + rk] = is_dead ? kRejected : 0u;
    }
    if (lane == 0) {
        ctl.resolved[b] = static_cast<unsigned>(ndead);
        ctl.nlive[b] = static_cast<unsigned>(N - ndead);
    }
}

// Node j's outputs of request b once every node is resolved (one wave); the
// caller holds the request's parents, tokens and slot ranks one node per lane
// (lanes past N: any values).
__device__ __forceinline__ void tree_finish(int p_in, int t_in, int rk_in, const int32_t *amax,
                                            const TreeCtl &ctl, int b, int N, int V,
                                            int32_t *__restrict__ accept_len, int32_t *__restrict__ path_nodes,
                                            int32_t *__restrict__ out_tokens, int32_t *__restrict__ status,
                                            int lane) {
    const long long base = static_cast<long long>(b) * N;
    const bool in = lane < N;
    const int p = in ? p_in : 0;
    const int t = in ? t_in : 0;
    const int rk = in ? rk_in : 0;
    const unsigned st = in ? shared_load(&ctl.state[base + rk]) : 0u;
    const int a = in && (st & kRowDone) ? shared_load(const_cast<int32_t *>(&amax[base + lane])) : -1;
    const bool bad_par = ballot(in && (lane == 0 ? p != -1 : (p < 0 || p >= lane))) != 0;
    const bool oor = ballot(in && lane > 0 && (t < 0 || t >= V)) != 0;
    if (bad_par) {
        for (int k = lane; k < N; k += kWave) {
            path_nodes[base + k] = -1;
            out_tokens[base + k] = -1;
        }
        if (lane == 0) {
            accept_len[b] = -1;
            if (status) status[b] = 2;
        }
        return;
    }
    // acceptance and depth by pointer jumping over the lanes
    const int pa = __shfl(a, lane == 0 ? 0 : p, kWave);  // argmax of the parent's row
    bool ok = lane == 0 ? true : (in && t == pa && pa >= 0);
    int dep = lane == 0 ? 0 : 1;
    int anc = lane == 0 ? 0 : p;
    for (int span = 1; span < N; span <<= 1) {
        const bool ok2 = __shfl(ok ? 1 : 0, anc, kWave) != 0;
        const int d2 = __shfl(dep, anc, kWave);
        const int a2 = __shfl(anc, anc, kWave);
        ok = ok && ok2;
        dep += d2;
        anc = a2;
    }
    // deepest accepted node, lowest index among equals (the root qualifies)
    const unsigned key = in && ok ? ((static_cast<unsigned>(dep) << 16) | (0xffffu - static_cast<unsigned>(lane))) : 0u;
    unsigned mk = key;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned y = static_cast<unsigned>(__shfl_xor(static_cast<int>(mk), o, kWave));
        mk = y > mk ? y : mk;
    }
    const int best = static_cast<int>(0xffffu - (uniform(mk) & 0xffffu));
    const int d = static_cast<int>(uniform(mk) >> 16);
    // the path: lane k (k < d) holds the ancestor of `best` at depth k + 1
    int node = best, walked = d;
    int mine = -1;
    while (walked > 0) {  // uniform: every lane walks the same chain
        if (lane == walked - 1) mine = node;
        node = __shfl(p, node, kWave);
        --walked;
    }
    const int mine_tok = __shfl(t, mine < 0 ? 0 : mine, kWave);
    const int bonus = __shfl(a, best, kWave);
    for (int k = lane; k < N; k += kWave) {
        path_nodes[base + k] = k < d ? mine : -1;
        out_tokens[base + k] = k < d ? mine_tok : (k == d ? bonus : -1);
    }
    if (lane == 0) {
        accept_len[b] = d;
        if (status) status[b] = oor ? 1 : 0;
    }
}

// Marks the nodes of `rej` rejected together with every node under them, and
// node `done` (-1: none) as having its row's argmax; counts the nodes whose
// state this changes from unresolved, and the wave whose count completes the
// request's N nodes writes its outputs.  The caller holds the request's
// parents, tokens and slot ranks one node per lane.
__device__ __forceinline__ void tree_mark(uint64_t rej, int done, int p, int t, int rk, const int32_t *amax,
                                          const TreeCtl &ctl, int b, int N, int V,
                                          int32_t *__restrict__ accept_len, int32_t *__restrict__ path_nodes,
                                          int32_t *__restrict__ out_tokens, int32_t *__restrict__ status,
                                          int lane) {
    const long long base = static_cast<long long>(b) * N;
    const bool in = lane < N;
    // close the rejection over the tree: a node under a rejected parent is rejected
    for (int it = 0; it < N; ++it) {
        const bool under = in && p >= 0 && p < lane && ((rej >> p) & 1ull);
        const uint64_t r2 = rej | ballot(under);
        if (r2 == rej) break;  // uniform
        rej = r2;
    }
    unsigned mark = 0;
    if (lane == done) mark |= kRowDone;
    if (in && ((rej >> lane) & 1ull)) mark |= kRejected;
    int newly = 0;
    if (mark) {
        const unsigned old = __hip_atomic_fetch_or(ctl.state + base + static_cast<unsigned>(rk), mark,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        newly = old == 0 ? 1 : 0;
    }
    const int cnt = __popcll(ballot(newly != 0));
    if (cnt == 0) return;
    wait_own_stores();
    unsigned before = 0;
    if (lane == 0)
        before = __hip_atomic_fetch_add(&ctl.resolved[b], static_cast<unsigned>(cnt), __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    before = uniform(static_cast<unsigned>(__shfl(static_cast<int>(before), 0, kWave)));
    if (before + static_cast<unsigned>(cnt) != static_cast<unsigned>(N)) return;
    tree_finish(p, t, rk, amax, ctl, b, N, V, accept_len, path_nodes, out_tokens, status, lane);
}

template <typename E, bool ALIGNED, int U>
__global__ __launch_bounds__(kBlock) void k_skip_tree(const typename E::storage *__restrict__ L,
                                                      const int32_t *__restrict__ tok,
                                                      const int32_t *__restrict__ par, int B, int N, int V,
                                                      int nvec, int segs, int rot, uint64_t *part_k,
                                                      int32_t *amax, TreeCtl ctl, int32_t *__restrict__ accept_len,
                                                      int32_t *__restrict__ path_nodes,
                                                      int32_t *__restrict__ out_tokens,
                                                      int32_t *__restrict__ status) {
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned wave = skip_wave_index();
    const unsigned per_slot = static_cast<unsigned>(B) * static_cast<unsigned>(segs);
    if (wave >= per_slot * static_cast<unsigned>(N)) return;
    const int slot = static_cast<int>(wave / per_slot);
    const unsigned rem = wave - static_cast<unsigned>(slot) * per_slot;
    const unsigned bslot = rem / static_cast<unsigned>(segs);
    const int sg = static_cast<int>(rem - bslot * static_cast<unsigned>(segs));
    const int b = skip_request(bslot, slot, B, rot);
    const long long base = static_cast<long long>(b) * N;
    // slots past the live count hold nodes the row samples rejected; the node
    // of a live slot may have been rejected since by a decision
    const unsigned nlive = uniform(ctl.nlive[b]);
    const int j = uniform(ctl.order[base + slot]);  // issued beside the state load
    if (static_cast<unsigned>(slot) >= nlive) return;
    // slot 0 holds the root, whose row is always needed
    if (slot > 0 && (uniform(shared_load(&ctl.state[base + slot])) & kRejected)) return;

    const long long row = base + j;
    int v0, v1;
    skip_segment(sg, nvec, segs, v0, v1);
    // the row's last segment decides node j's children: the request's
    // parents, tokens and slot ranks (one node per lane) are fetched before
    // the segment's loads
    const bool in = lane < N;
    int p = -1, t = 0, rk = 0;
    if (sg == segs - 1 && in) {
        p = par[base + lane];
        t = tok[base + lane];
        rk = ctl.rank[base + lane];
    }
    const uint64_t key = segment_argmax_chunked<E, ALIGNED, U, kGSkipChunks>(L + row * V, V, v0, v1, lane);
    // keys handed to the row's last segment as in the chain pass (the prep
    // launch zeroed them); a key never comes only if its wave found the node
    // already rejected, which this wave then finds too
    if (sg != segs - 1) {
        if (lane == 0) shared_store(&part_k[row * segs + sg], key);
        return;
    }
    uint64_t mk = key;
    bool complete = false;
    for (int it = 0; it < kSkipPollCap; ++it) {
        uint64_t m = 0;
        bool missing = false;
        for (int s = lane; s < segs - 1; s += kWave) {
            const uint64_t k = shared_load(&part_k[row * segs + s]);
            missing |= k == 0;
            m = k > m ? k : m;
        }
        if (ballot(missing) == 0) {
            mk = wave_max_u64(m > mk ? m : mk);
            complete = true;
            break;
        }
        if (uniform(shared_load(&ctl.state[base + slot])) & kRejected) return;
        __builtin_amdgcn_s_sleep(2);
    }
    if (!complete) return;  // never decide on part of a row
    const int a = uniform(argmax_key_index(mk));
    if (lane == 0) shared_store(&amax[row], a);
    wait_own_stores();
    // states as they stand, plus this row done and this row's mismatching children
    // the state word of each lane's node (the rank taken unsigned: its 64-bit
    // address then needs no value of it before the segment's loads)
    unsigned *st_word = ctl.state + base + static_cast<unsigned>(rk);
    unsigned st = in ? shared_load(st_word) : 0u;
    const uint64_t rej = ballot(in && ((st & kRejected) || (lane > 0 && p == j && t != a)));
    tree_mark(rej, j, p, t, rk, amax, ctl, b, N, V, accept_len, path_nodes, out_tokens, status, lane);
}

template <typename E, bool ALIGNED>
hipError_t skip_tree_t(const void *L, const int32_t *tok, const int32_t *par, int B, int N, int V,
                       const RowGeom &g, uint64_t *part_k, int32_t *amax, const TreeCtl &ctl,
                       int32_t *accept_len, int32_t *path_nodes, int32_t *out_tokens, int32_t *status,
                       hipStream_t s) {
    using T = typename E::storage;
    const long long nwaves = static_cast<long long>(N) * B * g.segs;
    const long long blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    return launch_kernel(k_skip_tree<E, ALIGNED, kGSkipVecsPerLane>, dim3(static_cast<unsigned>(blocks)),
                         dim3(kBlock), SV_TSKIP_LDS, s, static_cast<const T *>(L), tok, par, B, N, V, g.nvec, g.segs,
                         tree_rotation(B), part_k, amax, ctl, accept_len, path_nodes, out_tokens, status);
}

template <typename E, bool ALIGNED>
hipError_t skip_argmax_t(const void *L, const int32_t *drafts, int B, int K, int V, const RowGeom &g,
                         uint64_t *part_k, int32_t *amax, const SkipCtl &ctl, int32_t *accept_len,
                         int32_t *out_tokens, int32_t *status, hipStream_t s) {
    using T = typename E::storage;
    const long long nwaves = static_cast<long long>(K + 1) * B * g.segs;
    const long long blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    // the greedy chain always tests the rejection bits, and rotates where the
    // stochastic pass would test the finished flag (see greedy_rotation)
    const bool rotate = !skip_early(B, 1, V, sizeof(T));
    return launch_kernel(k_skip_argmax<E, ALIGNED, kGSkipVecsPerLane>, dim3(static_cast<unsigned>(blocks)),
                         dim3(kBlock), SV_GSKIP_LDS, s, static_cast<const T *>(L), drafts, B, K, V, g.nvec, g.segs,
                         part_k, amax, ctl, 1, greedy_rotation(B, rotate), accept_len, out_tokens, status);
}

template <typename E, bool ALIGNED>
hipError_t argmax_t(const void *L, long long rows, int V, const RowGeom &g, uint64_t *part_k,
                    hipStream_t s) {
    using T = typename E::storage;
    const long long nwaves = rows * g.segs;
    const long long blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    return launch_kernel(k_argmax<E, ALIGNED, kArgmaxVecsPerLane>, dim3(static_cast<unsigned>(blocks)),
                         dim3(kBlock), 0, s, static_cast<const T *>(L), nwaves, V, g.nvec, g.segs, part_k);
}

// Rows whose segment keys fit the LDS budget together (0: read them from global memory).
int stage_rows(int segs, int rows, size_t budget) {
    const size_t per_row = static_cast<size_t>(segs) * sizeof(uint64_t);
    if (per_row > budget) return 0;
    return static_cast<int>(std::min<size_t>(static_cast<size_t>(rows), budget / per_row));
}

}  // namespace

hipError_t launch_argmax(const void *L, long long rows, int V, const RowGeom &g, sv_dtype dt,
                         uint64_t *part_k, hipStream_t s) {
    if (dt == SV_BF16)
        return g.aligned ? argmax_t<BF16, true>(L, rows, V, g, part_k, s)
                         : argmax_t<BF16, false>(L, rows, V, g, part_k, s);
    return g.aligned ? argmax_t<F32, true>(L, rows, V, g, part_k, s)
                     : argmax_t<F32, false>(L, rows, V, g, part_k, s);
}

hipError_t launch_skip_match(const void *L, const int32_t *drafts, int B, int K, int V,
                             const RowGeom &g, sv_dtype dt, uint64_t *part_k, int32_t *amax,
                             void *ctl_base, int32_t *accept_len, int32_t *out_tokens,
                             int32_t *status, hipStream_t s) {
    SkipCtl ctl;
    // one workgroup per request clears its words and samples its rows
    skip_ctl_carve(ctl_base, B, K, &ctl);
    trace_select(-1);  // the preparing launch is not traced
#define SV_CP(E, A, T)                                                                                           \
    hipLaunchKernelGGL((k_chain_prep<E, A>), dim3(static_cast<unsigned>(B)), dim3(kBlock), 0, s,               \
                       static_cast<const T *>(L), drafts, B, K, V, g.nvec, g.segs, ctl, part_k, amax)
    if (dt == SV_BF16) {
        if (g.aligned)
            SV_CP(BF16, true, uint16_t);
        else
            SV_CP(BF16, false, uint16_t);
    } else {
        if (g.aligned)
            SV_CP(F32, true, float);
        else
            SV_CP(F32, false, float);
    }
#undef SV_CP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    trace_select(SV_K_SKIP_ARGMAX);
#define SV_SK(E, A) skip_argmax_t<E, A>(L, drafts, B, K, V, g, part_k, amax, ctl, accept_len, out_tokens, status, s)
    if (dt == SV_BF16) return g.aligned ? SV_SK(BF16, true) : SV_SK(BF16, false);
    return g.aligned ? SV_SK(F32, true) : SV_SK(F32, false);
#undef SV_SK
}

bool tree_skip_supported(int N) { return N <= kTreeSkipMaxN; }

size_t tree_ctl_bytes(int B, int N) { return sizeof(unsigned) * (3 * static_cast<size_t>(B) * N + 2 * static_cast<size_t>(B)); }

hipError_t launch_skip_tree(const void *L, const int32_t *node_tokens, const int32_t *parents, int B, int N,
                            int V, const RowGeom &g, sv_dtype dt, uint64_t *part_k, int32_t *amax,
                            void *ctl_base, int32_t *accept_len, int32_t *path_nodes, int32_t *out_tokens,
                            int32_t *status, hipStream_t s) {
    TreeCtl ctl;
    const size_t bn = static_cast<size_t>(B) * N;
    ctl.state = static_cast<unsigned *>(ctl_base);
    ctl.order = reinterpret_cast<int32_t *>(ctl.state + bn);
    ctl.rank = ctl.order + bn;
    ctl.resolved = reinterpret_cast<unsigned *>(ctl.rank + bn);
    ctl.nlive = ctl.resolved + B;
    trace_select(-1);  // the preparing launch is not traced
    const dim3 prep_grid(static_cast<unsigned>(B));
#define SV_TP(E, A, T)                                                                                          \
    hipLaunchKernelGGL((k_tree_prep<E, A>), prep_grid, dim3(kBlock), 0, s, static_cast<const T *>(L), parents, \
                       node_tokens, B, N, V, g.nvec, ctl, part_k, g.segs)
    if (dt == SV_BF16) {
        if (g.aligned)
            SV_TP(BF16, true, uint16_t);
        else
            SV_TP(BF16, false, uint16_t);
    } else {
        if (g.aligned)
            SV_TP(F32, true, float);
        else
            SV_TP(F32, false, float);
    }
#undef SV_TP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    trace_select(SV_K_SKIP_TREE);
#define SV_ST(E, A) skip_tree_t<E, A>(L, node_tokens, parents, B, N, V, g, part_k, amax, ctl, accept_len, path_nodes, out_tokens, status, s)
    if (dt == SV_BF16) return g.aligned ? SV_ST(BF16, true) : SV_ST(BF16, false);
    return g.aligned ? SV_ST(F32, true) : SV_ST(F32, false);
#undef SV_ST
}

hipError_t launch_match(const uint64_t *part_k, const int32_t *drafts, int B, int K, int V,
                        const RowGeom &g, int32_t *accept_len, int32_t *out_tokens, int32_t *status,
                        hipStream_t s) {
    const int lr = stage_rows(g.segs, K + 1, kMergeLdsBytes);
    const size_t lds = static_cast<size_t>(lr) * g.segs * sizeof(uint64_t) + sizeof(int) * static_cast<size_t>(K + 1);
    return launch_kernel(k_match, dim3(B), dim3(kBlock), lds, s, part_k, g.segs, lr, drafts, B, K, V,
                         accept_len, out_tokens, status);
}

hipError_t launch_tree(const uint64_t *part_k, const int32_t *node_tokens, const int32_t *parents,
                       int B, int N, int V, const RowGeom &g, int32_t *accept_len,
                       int32_t *path_nodes, int32_t *out_tokens, int32_t *status, hipStream_t s) {
    const size_t node_bytes = sizeof(int) * 6 * static_cast<size_t>(N);
    const size_t cap = 60 * 1024;
    const size_t budget = node_bytes < cap ? std::min<size_t>(kMergeLdsBytes, cap - node_bytes) : 0;
    const int lr = stage_rows(g.segs, N, budget);
    const size_t lds = static_cast<size_t>(lr) * g.segs * sizeof(uint64_t) + node_bytes;
    return launch_kernel(k_tree, dim3(B), dim3(kBlock), lds, s, part_k, g.segs, lr, node_tokens,
                         parents, B, N, V, accept_len, path_nodes, out_tokens, status);
}

}  // namespace sv
