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
//             segment to (max value, lowest index of that value).
//   k_match   one wave per request: merges segment partials in index order
//             (strictly greater replaces, so ties keep the lower segment) and
//             finds the first mismatch with a ballot.
//   k_tree    one workgroup per request: partial merge per node, parent-array
//             check in parallel, then the walk in index order (parents precede
//             children) and the path write-out.
#include <limits.h>

#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

template <typename E, bool ALIGNED, int U>
__global__ __launch_bounds__(kBlock) void k_argmax(const typename E::storage *__restrict__ L,
                                                   long long nwaves, int V, int nvec, int segs,
                                                   float *__restrict__ part_v,
                                                   int32_t *__restrict__ part_i) {
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
    if (lane == 0) {
        part_v[wave] = m;
        part_i[wave] = cand;
    }
}

// Argmax of one row from its segment partials (segments are in index order).
__device__ __forceinline__ int merge_argmax(const float *__restrict__ pv, const int32_t *__restrict__ pi,
                                            int segs) {
    float bv = pv[0];
    int bi = pi[0];
    for (int s = 1; s < segs; ++s) {
        const float v = pv[s];
        if (v > bv) {
            bv = v;
            bi = pi[s];
        }
    }
    return bi;
}

__global__ __launch_bounds__(kWave) void k_match(const float *__restrict__ part_v,
                                                 const int32_t *__restrict__ part_i, int segs,
                                                 const int32_t *__restrict__ drafts, int B, int K,
                                                 int V, int32_t *__restrict__ accept_len,
                                                 int32_t *__restrict__ out_tokens,
                                                 int32_t *__restrict__ status) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    int n = -1, a_n = -1;
    bool bad = false;
    for (int i0 = 0; i0 <= K; i0 += kWave) {
        const int i = i0 + lane;
        int a = -1;
        bool stop = false;
        if (i <= K) {
            const long long g = (static_cast<long long>(b) * (K + 1) + i) * segs;
            a = merge_argmax(part_v + g, part_i + g, segs);
            if (i < K) {
                const int x = drafts[static_cast<long long>(b) * K + i];
                if (x < 0 || x >= V) bad = true;
                stop = x != a;
            } else {
                stop = true;  // the bonus row ends every chain
            }
        }
        const uint64_t mk = ballot(stop);
        if (n < 0 && mk != 0) {  // uniform: every lane takes this branch together
            const int l = first_lane(mk);
            n = i0 + l;
            a_n = __shfl(a, l, kWave);
        }
    }
    const bool any_bad = ballot(bad) != 0;
    int32_t *tok = out_tokens + static_cast<long long>(b) * (K + 1);
    for (int i = lane; i <= K; i += kWave)
        tok[i] = i < n ? drafts[static_cast<long long>(b) * K + i] : (i == n ? a_n : -1);
    if (lane == 0) {
        accept_len[b] = n;
        if (status) status[b] = any_bad ? 1 : 0;
    }
}

__global__ __launch_bounds__(kBlock) void k_tree(const float *__restrict__ part_v,
                                                 const int32_t *__restrict__ part_i, int segs,
                                                 const int32_t *__restrict__ node_tokens,
                                                 const int32_t *__restrict__ parents, int B, int N,
                                                 int V, int32_t *__restrict__ accept_len,
                                                 int32_t *__restrict__ path_nodes,
                                                 int32_t *__restrict__ out_tokens,
                                                 int32_t *__restrict__ status) {
    extern __shared__ int smem[];
    int *s_a = smem;          // argmax of each node's row
    int *s_par = s_a + N;     // parents
    int *s_tok = s_par + N;   // node tokens
    int *s_ok = s_tok + N;    // accepted flag
    int *s_dep = s_ok + N;    // depth
    int *s_path = s_dep + N;  // chosen path, depth 1 first
    __shared__ int s_bad, s_oor, s_best, s_d;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_bad = 0;
        s_oor = 0;
    }
    __syncthreads();
    const long long base = static_cast<long long>(b) * N;
    for (int j = tid; j < N; j += blockDim.x) {
        const long long g = (base + j) * segs;
        s_a[j] = merge_argmax(part_v + g, part_i + g, segs);
        const int p = parents[base + j];
        const int t = node_tokens[base + j];
        s_par[j] = p;
        s_tok[j] = t;
        if (j == 0 ? p != -1 : (p < 0 || p >= j)) atomicOr(&s_bad, 1);
        if (j > 0 && (t < 0 || t >= V)) atomicOr(&s_oor, 1);
    }
    __syncthreads();
    if (s_bad) {
        for (int k = tid; k < N; k += blockDim.x) {
            path_nodes[base + k] = -1;
            out_tokens[base + k] = -1;
        }
        if (tid == 0) {
            accept_len[b] = -1;
            if (status) status[b] = 2;
        }
        return;
    }
    if (tid == 0) {
        s_ok[0] = 1;
        s_dep[0] = 0;
        int best = 0;
        for (int j = 1; j < N; ++j) {
            const int p = s_par[j];
            const int ok = s_ok[p] && s_tok[j] == s_a[p];
            const int d = s_dep[p] + 1;
            s_ok[j] = ok;
            s_dep[j] = d;
            if (ok && d > s_dep[best]) best = j;
        }
        const int d = s_dep[best];
        for (int j = best, k = d - 1; j != 0; j = s_par[j], --k) s_path[k] = j;
        s_best = best;
        s_d = d;
    }
    __syncthreads();
    const int d = s_d;
    for (int k = tid; k < N; k += blockDim.x) {
        path_nodes[base + k] = k < d ? s_path[k] : -1;
        out_tokens[base + k] = k < d ? s_tok[s_path[k]] : (k == d ? s_a[s_best] : -1);
    }
    if (tid == 0) {
        accept_len[b] = d;
        if (status) status[b] = s_oor ? 1 : 0;
    }
}

template <typename E, bool ALIGNED>
hipError_t argmax_t(const void *L, long long rows, int V, const RowGeom &g, float *part_v,
                    int32_t *part_i, hipStream_t s) {
    using T = typename E::storage;
    const long long nwaves = rows * g.segs;
    const long long blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    k_argmax<E, ALIGNED, kStreamVecsPerLane><<<dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s>>>(
        static_cast<const T *>(L), nwaves, V, g.nvec, g.segs, part_v, part_i);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_argmax(const void *L, long long rows, int V, const RowGeom &g, sv_dtype dt,
                         float *part_v, int32_t *part_i, hipStream_t s) {
    if (dt == SV_BF16)
        return g.aligned ? argmax_t<BF16, true>(L, rows, V, g, part_v, part_i, s)
                         : argmax_t<BF16, false>(L, rows, V, g, part_v, part_i, s);
    return g.aligned ? argmax_t<F32, true>(L, rows, V, g, part_v, part_i, s)
                     : argmax_t<F32, false>(L, rows, V, g, part_v, part_i, s);
}

hipError_t launch_match(const float *part_v, const int32_t *part_i, const int32_t *drafts, int B,
                        int K, int V, const RowGeom &g, int32_t *accept_len, int32_t *out_tokens,
                        int32_t *status, hipStream_t s) {
    k_match<<<dim3(B), dim3(kWave), 0, s>>>(part_v, part_i, g.segs, drafts, B, K, V, accept_len,
                                            out_tokens, status);
    return hipGetLastError();
}

hipError_t launch_tree(const float *part_v, const int32_t *part_i, const int32_t *node_tokens,
                       const int32_t *parents, int B, int N, int V, const RowGeom &g,
                       int32_t *accept_len, int32_t *path_nodes, int32_t *out_tokens,
                       int32_t *status, hipStream_t s) {
    const size_t lds = sizeof(int) * 6 * static_cast<size_t>(N);
    k_tree<<<dim3(B), dim3(kBlock), lds, s>>>(part_v, part_i, g.segs, node_tokens, parents, B, N,
                                              V, accept_len, path_nodes, out_tokens, status);
    return hipGetLastError();
}

}  // namespace sv
