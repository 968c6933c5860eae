// sv_sample.hip -- stochastic chain verification (speculative sampling).
//
// What is computed follows the speculative-decoding tutorial page, sections
// "一轮推测解码究竟发生什么" (accept draft x_i with probability
// min(1, p_i(x_i)/q_i(x_i)), discard every later draft at the first rejection,
// then draw one target token: from the corrected residual at the rejected
// position, or from the next-position distribution when all drafts pass) and
// "为什么“猜错再改”不会偏离目标分布" (residual norm(max(0, p - q))).
//
// Kernels, all on the caller's stream:
//   k_rowstats     one streaming pass over every target row [B,K+1,V] and draft
//                  row [B,K,V]; each wave reduces a segment of a row to a
//                  partial (R, s) with s = sum 2^(x c - R), c = log2(e)/T.
//   k_accept       one workgroup per request: stages the partials of its 2K+1
//                  rows in LDS, merges each row (a wave merges four rows at
//                  once) into
//                  L2 = log2 sum_v 2^(x c), gathers L[x_i] for every draft,
//                  forms p_i(x_i)/q_i(x_i) in fp64 and finds the first
//                  rejection; writes accept_len, the accepted tokens, lse.
//   k_resid_mass   for the one row (pair) each request draws from, the mass of
//                  max(0, p - q) (or p for the bonus) per 64-vector tile.
//   k_resid_select one wave per request: prefix over tile masses, then over
//                  lanes of the chosen tile, then over the elements of the
//                  chosen lane; writes the drawn token.
//   k_skip_stats   without lse outputs and for K <= 31, k_rowstats and the
//                  acceptance in one launch that does not read the rows of
//                  positions after each request's first rejection (protocol in
//                  sv_skip.hpp); the residual kernels then run as above.
//   k_merge_parts  the fused LM-head form's many 128-column partials per
//                  target row merged to one per row before k_accept; there
//                  the residual kernels read the re-formed fp32 target row
//                  beside the draft row in its own type.
//
// Precision: per-element exponentials run in fp32 on v_exp_f32 with the
// exponent formed by two fused multiply-adds against c = c_hi + c_lo, so the
// temperature scale carries no systematic rounding; every accumulation across
// elements, the row merges, the acceptance ratios and the running masses of the
// inverse CDF are fp64.
#include <algorithm>
#include <type_traits>

#include "sv_device.hpp"
#include "sv_internal.hpp"
#include "sv_skip.hpp"

namespace sv {
namespace {

constexpr double kLn2 = 0.6931471805599453094172321214581766;

// The draw's per-row constants (used by the residual kernels): half the
// probability of logit x in a row with log2-normaliser L2 is 2^(x c - R),
// R = L2 + 1.  With R = R_hi + R_lo, R_hi the nearest float, the kernels form
// t(x) = x c_lo + (x c_hi - R_hi) with two fmas; 2^t(x) then differs from the
// half-probability by the factor 2^R_lo, the same for a whole row.  The draw
// only compares masses of one row pair, so the target row's factor is carried
// over to the draft row's as r = 2^(Rq_lo - Rp_lo), and the common factor
// that remains is dropped.  A row with no finite logit (R = -inf) keeps
// R_lo = 0.
__device__ __forceinline__ void draw_constants(ResidParam &P) {
    const double Rp = P.L2p + 1.0, Rq = P.mode ? P.L2q + 1.0 : 1.0;
    P.Rp_hi = static_cast<float>(Rp);
    P.Rq_hi = static_cast<float>(Rq);
    const double lp = isfinite(Rp) ? Rp - static_cast<double>(P.Rp_hi) : 0.0;
    const double lq = isfinite(Rq) ? Rq - static_cast<double>(P.Rq_hi) : 0.0;
    P.r = P.mode ? static_cast<float>(exp2(lq - lp)) : 1.0f;
}

// ---- S1: per-segment row statistics ---------------------------------------------

// One wave's (R, s) over vectors [v0, v1) of a row: R = fp32(max * c_hi) and
// s = sum 2^(x c - R) with the exponent formed by two fused multiply-adds.
// A segment that is all -inf yields (-inf, 0).
template <typename E, bool ALIGNED, int U>
__device__ __forceinline__ void segment_stats(const typename E::storage *__restrict__ base, int V,
                                              int v0, int v1, float c_hi, float c_lo, int lane,
                                              float &R, double &s) {
    constexpr int P = E::kPerVec;
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
    R = -__builtin_huge_valf();
    s = 0.0;
    if (m != -__builtin_huge_valf()) {
        R = m * c_hi;
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float x[P];
            st[k].get(x);
#pragma unroll
            for (int e = 0; e < P; ++e) x[e] = fast_exp2(fmaf(x[e], c_lo, fmaf(x[e], c_hi, -R)));
            s += static_cast<double>(pairwise_sum(x));
        }
        s = wave_sum(s);
    }
}

// (R, s) of vectors [v0, v1) walked in chunks of 64*U vectors, the next
// chunk's loads issued before the current chunk is summed.  Each chunk gets
// its own reference R_k; the chunks are combined in fp64 at the end.
template <typename E, bool ALIGNED, int U, int CH>
__device__ __forceinline__ void segment_stats_chunked(const typename E::storage *__restrict__ base, int V,
                                                      int v0, int v1, float c_hi, float c_lo, int lane,
                                                      float &R, double &s) {
    constexpr int P = E::kPerVec;
    float Rk[CH];
    double sk[CH];
    Staged<E, ALIGNED> a[U], b[U];
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
    auto sum = [&](const Staged<E, ALIGNED>(&st)[U], int ch) {
        float m = -__builtin_huge_valf();
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float x[P];
            st[k].get(x);
#pragma unroll
            for (int e = 0; e < P; ++e) m = fmaxf(m, x[e]);
        }
        m = wave_max(m);
        float r = -__builtin_huge_valf();
        double t = 0.0;
        if (m != -__builtin_huge_valf()) {
            r = m * c_hi;
#pragma unroll
            for (int k = 0; k < U; ++k) {
                float x[P];
                st[k].get(x);
#pragma unroll
                for (int e = 0; e < P; ++e) x[e] = fast_exp2(fmaf(x[e], c_lo, fmaf(x[e], c_hi, -r)));
                t += static_cast<double>(pairwise_sum(x));
            }
        }
        Rk[ch] = r;
        sk[ch] = t;
    };
    constexpr int step = kWave * U;
    load(a, v0);
#pragma unroll
    for (int ch = 0; ch < CH; ch += 2) {
        if (ch + 1 < CH) load(b, v0 + (ch + 1) * step);
        sum(a, ch);
        if (ch + 2 < CH) load(a, v0 + (ch + 2) * step);
        if (ch + 1 < CH) sum(b, ch + 1);
    }
    float Rm = -__builtin_huge_valf();
#pragma unroll
    for (int ch = 0; ch < CH; ++ch) Rm = fmaxf(Rm, Rk[ch]);
    double t = 0.0;
    if (Rm != -__builtin_huge_valf()) {
#pragma unroll
        for (int ch = 0; ch < CH; ++ch)
            if (sk[ch] > 0.0) t += sk[ch] * exp2(static_cast<double>(Rk[ch]) - static_cast<double>(Rm));
    }
    R = Rm;
    s = wave_sum(t);
}

template <typename E, bool ALIGNED, int U>
__global__ __launch_bounds__(kBlock) void k_rowstats(
    const typename E::storage *__restrict__ tgt, const typename E::storage *__restrict__ drf,
    long long rows_t, long long nwaves, int V, int nvec, int segs, float c_hi, float c_lo,
    float *__restrict__ part_R, double *__restrict__ part_s) {
    const int lane = threadIdx.x & (kWave - 1);
    const long long wave = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (wave >= nwaves) return;
    const long long row = wave / segs;
    const int seg = static_cast<int>(wave - row * segs);
    const typename E::storage *base =
        row < rows_t ? tgt + row * static_cast<long long>(V) : drf + (row - rows_t) * static_cast<long long>(V);
    const int v0 = static_cast<int>((static_cast<long long>(seg) * nvec) / segs);
    const int v1 = static_cast<int>((static_cast<long long>(seg + 1) * nvec) / segs);
    float R;
    double sum;
    segment_stats<E, ALIGNED, U>(base, V, v0, v1, c_hi, c_lo, lane, R, sum);
    if (lane == 0) {
        part_R[wave] = R;
        part_s[wave] = sum;
    }
}

// ---- S2/S3: merge, gather, acceptance scan ----------------------------------------

// One partial per row out of `segs` per row: (Rm, sum_k s_k 2^(R_k - Rm)), Rm
// the largest R_k, summed lane-strided and then across the wave exactly as
// k_accept merges a row.  k_accept merging that single partial then finds the
// same L2 = Rm + log2(sum) bit for bit.  For rows with many segments (the
// fused projection's 128-column partials): one wave per row.  Each lane
// loads kMergeUnroll of its partials before it uses any of them (the loop is
// otherwise one memory latency per partial); the additions keep their order.
constexpr int kMergeUnroll = 8;
__global__ __launch_bounds__(kBlock) void k_merge_parts(const float *__restrict__ R, const double *__restrict__ S,
                                                        long long rows, int segs, float *__restrict__ outR,
                                                        double *__restrict__ outS) {
    constexpr int U = kMergeUnroll;
    const int lane = threadIdx.x & (kWave - 1);
    const long long row = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float *pR = R + row * segs;
    const double *pS = S + row * segs;
    const float ninf = -__builtin_huge_valf();
    float Rm = ninf;
    for (int sg0 = lane; sg0 < segs; sg0 += U * kWave) {
        float r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = sg0 + u * kWave < segs ? pR[sg0 + u * kWave] : ninf;
#pragma unroll
        for (int u = 0; u < U; ++u) Rm = fmaxf(Rm, r[u]);
    }
    Rm = wave_max(Rm);
    double acc = 0.0;
    if (Rm != ninf) {
        for (int sg0 = lane; sg0 < segs; sg0 += U * kWave) {
            float r[U];
            double ss[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int sg = sg0 + u * kWave;
                r[u] = sg < segs ? pR[sg] : ninf;
                ss[u] = sg < segs ? pS[sg] : 0.0;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ss[u] > 0.0) acc += ss[u] * exp2(static_cast<double>(r[u]) - static_cast<double>(Rm));
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
        outR[row] = Rm;
        outS[row] = acc;
    }
}

// FUSED: the target rows were never written (their partials come from the
// LM-head projection, which also kept the logit at each draft in xlog), and
// the row each request draws from is formed afterwards at row b of a
// per-request buffer; its draft row is read where it lies.
template <typename E, bool FUSED>
__global__ __launch_bounds__(kBlock) void k_accept(
    const typename E::storage *__restrict__ tgt, const typename E::storage *__restrict__ drf,
    const int32_t *__restrict__ drafts, const float *__restrict__ ua, const float *__restrict__ us,
    int B, int K, int V, PartRows pt, PartRows pd, int lds_rows, double c, const float *__restrict__ xlog,
    double *__restrict__ L2out, int32_t *__restrict__ accept_len, int32_t *__restrict__ out_tokens,
    float *__restrict__ lse_t, float *__restrict__ lse_d, int32_t *__restrict__ status,
    ResidParam *__restrict__ rp) {
    // LDS: the 2K+1 row log2-normalisers, then staged partials of lds_rows rows
    // (staging only when target and draft rows have the same segment count)
    extern __shared__ __align__(16) unsigned char smem[];
    const int nrows = 2 * K + 1;
    const int segs = pt.segs;
    double *sL2 = reinterpret_cast<double *>(smem);
    double *stS = sL2 + nrows;
    float *stR = reinterpret_cast<float *>(stS + static_cast<size_t>(lds_rows) * segs);
    const int b = blockIdx.x;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & (kWave - 1);
    const double inf = __builtin_huge_val();
    // partials of row r of this request: target rows 0..K, then draft rows
    // (the two argument structs' fields taken as scalars once, so that picking
    // a row selects between scalars rather than loading through a pointer)
    const float *const ptR = pt.R, *const pdR = pd.R;
    const double *const ptS = pt.s, *const pdS = pd.s;
    const int tsegs = pt.segs, dsegs = pd.segs;
    auto row_R = [&](int r) {
        return r <= K ? ptR + (static_cast<long long>(b) * (K + 1) + r) * tsegs
                      : pdR + (static_cast<long long>(b) * K + (r - K - 1)) * dsegs;
    };
    auto row_s = [&](int r) {
        return r <= K ? ptS + (static_cast<long long>(b) * (K + 1) + r) * tsegs
                      : pdS + (static_cast<long long>(b) * K + (r - K - 1)) * dsegs;
    };
    // the target logit at draft i (its row scores draft i), as stored bits
    auto tgt_bits = [&](int i, int x) {
        if constexpr (FUSED)
            return __float_as_uint(xlog[static_cast<long long>(b) * (K + 1) + i]);
        else
            return storage_bits(tgt[(static_cast<long long>(b) * (K + 1) + i) * V + x]);
    };
    auto tgt_value = [&](unsigned u) {
        if constexpr (FUSED)
            return __uint_as_float(u);
        else
            return from_bits<E>(u);
    };

    // The drafts and the two logits each one is scored with, fetched for the
    // first 64 positions while the partials are merged (kept as loaded, and
    // converted only where they are used, so that nothing waits for them
    // before the merge).
    const int32_t *xb = drafts + static_cast<long long>(b) * K;
    int x0 = -1;
    unsigned xp0b = 0, xq0b = 0;
    if (tid < K) {
        x0 = xb[tid];
        if (x0 >= 0 && x0 < V) {
            xp0b = tgt_bits(tid, x0);
            xq0b = storage_bits(drf[(static_cast<long long>(b) * K + tid) * V + x0]);
        }
    }

    // 1. row normalisers L2 = Rmax + log2 sum_s s_s 2^(R_s - Rmax)
    const int chunk = lds_rows > 0 ? lds_rows : nrows;
    for (int r0 = 0; r0 < nrows; r0 += chunk) {
        const int nr = min(chunk, nrows - r0);
        if (lds_rows > 0) {
            // kStage loads per thread issued before any is stored
            constexpr int kStage = 4;
            for (int i0 = tid; i0 < nr * segs; i0 += kStage * kBlock) {
                float sr[kStage];
                double ssv[kStage];
#pragma unroll
                for (int u = 0; u < kStage; ++u) {
                    const int i = i0 + u * kBlock;
                    if (i < nr * segs) {
                        const int rr = i / segs, sg = i - rr * segs;
                        sr[u] = row_R(r0 + rr)[sg];
                        ssv[u] = row_s(r0 + rr)[sg];
                    }
                }
#pragma unroll
                for (int u = 0; u < kStage; ++u) {
                    const int i = i0 + u * kBlock;
                    if (i < nr * segs) {
                        stR[i] = sr[u];
                        stS[i] = ssv[u];
                    }
                }
            }
            __syncthreads();
        }
        // a wave merges kMergeILP rows at once (rows wid, wid + 4, ...): the
        // rows are independent, so their loads, exponentials and reductions
        // overlap; each row is still reduced in the same order
        constexpr int kMergeILP = 4;
        for (int rb = wid; rb < nr; rb += kMergeILP * kWavesPerBlock) {
            const float *pR[kMergeILP];
            const double *pS[kMergeILP];
            int ns[kMergeILP];
            bool ok[kMergeILP];
            float Rm[kMergeILP];
            double acc[kMergeILP];
#pragma unroll
            for (int q = 0; q < kMergeILP; ++q) {
                const int rr = rb + q * kWavesPerBlock;
                ok[q] = rr < nr;
                const int rc = ok[q] ? rr : rb;
                if (lds_rows > 0) {
                    pR[q] = stR + rc * segs;
                    pS[q] = stS + rc * segs;
                    ns[q] = segs;
                } else {
                    pR[q] = row_R(r0 + rc);
                    pS[q] = row_s(r0 + rc);
                    ns[q] = r0 + rc <= K ? tsegs : dsegs;
                }
                Rm[q] = -__builtin_huge_valf();
                for (int sg = lane; sg < ns[q]; sg += kWave) Rm[q] = fmaxf(Rm[q], pR[q][sg]);
            }
#pragma unroll
            for (int q = 0; q < kMergeILP; ++q) {
                Rm[q] = wave_max(Rm[q]);
                acc[q] = 0.0;
                if (Rm[q] != -__builtin_huge_valf()) {
                    for (int sg = lane; sg < ns[q]; sg += kWave) {
                        const double ss = pS[q][sg];
                        if (ss > 0.0)
                            acc[q] += ss * exp2(static_cast<double>(pR[q][sg]) - static_cast<double>(Rm[q]));
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < kMergeILP; ++q) {
                acc[q] = wave_sum(acc[q]);
                const int r = r0 + rb + q * kWavesPerBlock;
                const double l2 = acc[q] > 0.0 ? static_cast<double>(Rm[q]) + log2(acc[q]) : -inf;
                if (ok[q] && lane == 0) {
                    sL2[r] = l2;
                    L2out[static_cast<long long>(b) * nrows + r] = l2;
                    if (r <= K) {
                        if (lse_t) lse_t[static_cast<long long>(b) * (K + 1) + r] = static_cast<float>(l2 * kLn2);
                    } else if (lse_d) {
                        lse_d[static_cast<long long>(b) * K + (r - K - 1)] = static_cast<float>(l2 * kLn2);
                    }
                }
            }
        }
        __syncthreads();
    }
    if (wid != 0) return;
    // the prefetched logits are needed from here on
    asm volatile("" : "+v"(xp0b), "+v"(xq0b));
    const float xp0 = tgt_value(xp0b), xq0 = from_bits<E>(xq0b);

    // 2. p_i(x_i) / q_i(x_i) for every position at once; the first failing test wins.
    int n = K;
    bool bad = false;
    for (int i0 = 0; i0 < K; i0 += kWave) {
        const int i = i0 + lane;
        bool rej = false;
        if (i < K) {
            const int x = i0 == 0 ? x0 : xb[i];
            double r = 0.0;
            if (x >= 0 && x < V) {
                const double xp = i0 == 0 ? xp0 : tgt_value(tgt_bits(i, x));
                const double xq = i0 == 0 ? xq0 : to_f32(drf[(static_cast<long long>(b) * K + i) * V + x]);
                const double px = exp2(xp * c - sL2[i]);
                const double qx = exp2(xq * c - sL2[K + 1 + i]);
                r = qx == 0.0 ? inf : px / qx;
            } else {
                bad = true;
            }
            const double u = static_cast<double>(ua[static_cast<long long>(b) * K + i]);
            rej = !(u < r);
        }
        const uint64_t mk = ballot(rej);
        if (mk != 0 && n == K) n = i0 + first_lane(mk);
    }
    const bool any_bad = ballot(bad) != 0;

    int32_t *tok = out_tokens + static_cast<long long>(b) * (K + 1);
    for (int i = lane; i <= K; i += kWave) tok[i] = i < n ? (i < kWave ? x0 : xb[i]) : -1;
    if (lane == 0) {
        accept_len[b] = n;
        if (status) status[b] = any_bad ? 1 : 0;
        ResidParam P;
        P.pos = n;
        P.u = static_cast<double>(us[static_cast<long long>(b) * (K + 1) + n]);
        P.row_p = FUSED ? b : static_cast<long long>(b) * (K + 1) + n;
        P.L2p = sL2[n];
        if (n < K) {
            P.mode = 1;
            P.row_q = static_cast<long long>(b) * K + n;
            P.L2q = sL2[K + 1 + n];
        } else {
            P.mode = 0;
            P.row_q = 0;
            P.L2q = 0.0;
        }
        draw_constants(P);
        rp[b] = P;
    }
}

// ---- S4/S5: the drawn token -------------------------------------------------------

// Per-request constants of the draw (see draw_constants): element masses are
// taken up to a factor common to the request's row pair, which the inverse
// CDF over them does not see.
struct Draw {
    float c_hi, c_lo, Rp, Rq, r;
    int mode;
};

__device__ __forceinline__ Draw make_draw(const ResidParam &P, float c_hi, float c_lo, int mode) {
    Draw d;
    d.c_hi = c_hi;
    d.c_lo = c_lo;
    d.Rp = P.Rp_hi;
    d.Rq = P.Rq_hi;
    d.r = P.r;
    d.mode = mode;
    return d;
}

// 2^t(x), t(x) = x c_lo + (x c_hi - R): the first fma cancels exactly
// against R, the second adds the low part of the scale (c_lo > 0, so -inf
// stays -inf).
__device__ __forceinline__ float half_prob(float x, const Draw &D, float R) {
    return fast_exp2(fmaf(x, D.c_lo, fmaf(x, D.c_hi, -R)));
}

// Mass of each element of one vector, up to the row pair's common factor:
// max(0, p - q) (PAIR) or p.  A pair's element mass is below 1 (the halving
// in draw_constants), so max(0, .) is the clamp to [0, 1], which the
// hardware applies to the fma's result at no cost (a NaN, as from a row with
// no finite logit, clamps to 0 as fmaxf would make it).
template <bool PAIR, int P>
__device__ __forceinline__ void masses(const float (&xp)[P], const float (&xq)[P], const Draw &D,
                                       float (&d)[P]) {
#pragma unroll
    for (int e = 0; e < P; ++e) {
        const float p = half_prob(xp[e], D, D.Rp);
        if (PAIR)
            d[e] = __builtin_amdgcn_fmed3f(fmaf(p, D.r, -half_prob(xq[e], D, D.Rq)), 0.0f, 1.0f);
        else
            d[e] = p;
    }
}

template <int P>
__device__ __forceinline__ void masses(const float (&xp)[P], const float (&xq)[P], const Draw &D,
                                       float (&d)[P]) {
    if (D.mode)
        masses<true>(xp, xq, D, d);
    else
        masses<false>(xp, xq, D, d);
}

template <int P>
__device__ __forceinline__ double lane_total(const float (&d)[P]) {
    float t[P];
#pragma unroll
    for (int e = 0; e < P; ++e) t[e] = d[e];
    return static_cast<double>(pairwise_sum(t));
}

// The draft row's stager: the target row's own type, or a bf16 draft row read
// four elements at a time beside fp32 target rows.
template <typename E, typename EQ, bool ALIGNED>
using DraftStaged =
    typename std::conditional<std::is_same<E, EQ>::value, Staged<E, ALIGNED>, Staged4<EQ, ALIGNED>>::type;

// Tiles [t_begin, t_end) of one request's draw row(s), walked in groups of G
// with the next group's loads in flight while one group is summed.  Every
// load of the aligned form is issued unconditionally, so that the wait before
// a group's sums covers that group's loads only: a vector past the row's end
// re-reads the row's last vector, and its masses are zeroed afterwards.
template <typename E, typename EQ, bool ALIGNED, int G, bool PAIR>
__device__ __forceinline__ void resid_tiles(const typename E::storage *__restrict__ prow,
                                            const typename EQ::storage *__restrict__ qrow, int V, int nvec,
                                            int t_begin, int t_end, const Draw &D, int lane,
                                            double *__restrict__ out) {
    constexpr int P = E::kPerVec;
    using QS = DraftStaged<E, EQ, ALIGNED>;
    auto load = [&](Staged<E, ALIGNED>(&sp)[G], QS(&sq)[G], int t0) {
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const int j = min((t0 + k) * kWave + lane, nvec - 1);
            sp[k].load(prow, V, j);
            if (PAIR) sq[k].load(qrow, V, j);
        }
    };
    // the tiles' totals (only the totals are kept), two tiles per reduction
    auto sum = [&](const Staged<E, ALIGNED>(&sp)[G], const QS(&sq)[G], int t0) {
        double part[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
            const int t = t0 + k;
            part[k] = 0.0;
            if (t < t_end) {  // uniform across the wave
                float xp[P], xq[P], d[P];
                sp[k].get(xp);
                if (PAIR) sq[k].get(xq);
                masses<PAIR>(xp, xq, D, d);
                const float lt = pairwise_sum(d);
                part[k] = t * kWave + lane < nvec ? static_cast<double>(lt) : 0.0;  // else a re-read past the row's end
            }
        }
#pragma unroll
        for (int k = 0; k < G; k += 2) {
            const double tot = wave_sum_pair(part[k], k + 1 < G ? part[k + 1] : 0.0);
            if (lane == 0 && t0 + k < t_end) out[t0 + k] = tot;
            if (lane == kWave / 2 && k + 1 < G && t0 + k + 1 < t_end) out[t0 + k + 1] = tot;
        }
    };
    Staged<E, ALIGNED> ap[G], bp[G];
    QS aq[G], bq[G];
    int t0 = t_begin;
    load(ap, aq, t0);
    // whole pairs of groups while another group follows them
    for (; t0 + 2 * G < t_end; t0 += 2 * G) {
        load(bp, bq, t0 + G);
        sum(ap, aq, t0);
        load(ap, aq, t0 + 2 * G);
        sum(bp, bq, t0 + G);
    }
    if (t0 + G < t_end) {
        load(bp, bq, t0 + G);
        sum(ap, aq, t0);
        sum(bp, bq, t0 + G);
    } else {
        sum(ap, aq, t0);
    }
}

// Residual (or bonus) mass of each 64-vector tile of the row each request
// draws from.  A wave owns `tpw` consecutive tiles of one request; its
// position, request and draw mode are scalars.
template <typename E, typename EQ, bool ALIGNED, int G>
__global__ __launch_bounds__(kBlock) void k_resid_mass(
    const typename E::storage *__restrict__ tgt, const typename EQ::storage *__restrict__ drf,
    int B, int V, int nvec, int ntiles, int wpr, int tpw, float c_hi, float c_lo,
    const ResidParam *__restrict__ rp, double *__restrict__ tile_mass) {
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned wave = blockIdx.x * static_cast<unsigned>(kWavesPerBlock) + uniform(static_cast<unsigned>(threadIdx.x >> 6));
    if (wave >= static_cast<unsigned>(B) * static_cast<unsigned>(wpr)) return;
    const int b = static_cast<int>(wave / static_cast<unsigned>(wpr));
    const int w = static_cast<int>(wave - static_cast<unsigned>(b) * static_cast<unsigned>(wpr));
    const ResidParam &Pm = rp[b];
    const Draw D = make_draw(Pm, c_hi, c_lo, uniform(Pm.mode));
    const typename E::storage *prow = tgt + Pm.row_p * static_cast<long long>(V);
    const int t_begin = w * tpw;
    const int t_end = min(ntiles, t_begin + tpw);
    double *out = tile_mass + static_cast<long long>(b) * ntiles;
    if (D.mode)
        resid_tiles<E, EQ, ALIGNED, G, true>(prow, drf + Pm.row_q * static_cast<long long>(V), V, nvec, t_begin,
                                             t_end, D, lane, out);
    else
        resid_tiles<E, EQ, ALIGNED, G, false>(prow, nullptr, V, nvec, t_begin, t_end, D, lane, out);
}

template <typename E, typename EQ, bool ALIGNED>
__global__ __launch_bounds__(kWave) void k_resid_select(
    const typename E::storage *__restrict__ tgt, const typename EQ::storage *__restrict__ drf,
    int B, int K, int V, int nvec, int ntiles, float c_hi, float c_lo,
    const ResidParam *__restrict__ rp, double *__restrict__ tile_mass, int32_t *__restrict__ out_tokens) {
    constexpr int P = E::kPerVec;
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const ResidParam Pm = rp[b];
    Draw D = make_draw(Pm, c_hi, c_lo, Pm.mode);
    const typename E::storage *prow = tgt + Pm.row_p * static_cast<long long>(V);
    const typename EQ::storage *qrow = D.mode ? drf + Pm.row_q * static_cast<long long>(V) : nullptr;
    double *tm = tile_mass + static_cast<long long>(b) * ntiles;
    int32_t *dst = out_tokens + static_cast<long long>(b) * (K + 1) + Pm.pos;

    // tiles [lt0, lt1) belong to this lane; prefix over lanes in tile order.
    // The lane's first kSelRegs masses are loaded at once into registers (the
    // rest, for rows of more than 64 kSelRegs tiles, one by one) and summed in
    // tile order.
    constexpr int kSelRegs = 16;
    const int tpl = (ntiles + kWave - 1) / kWave;
    const int lt0 = min(ntiles, lane * tpl), lt1 = min(ntiles, lt0 + tpl);
    double tmr[kSelRegs];
    auto lane_masses = [&]() {
#pragma unroll
        for (int k = 0; k < kSelRegs; ++k) tmr[k] = lt0 + k < lt1 ? tm[lt0 + k] : 0.0;
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < kSelRegs; ++k) acc += tmr[k];
        for (int t = lt0 + kSelRegs; t < lt1; ++t) acc += tm[t];
        return acc;
    };
    double ls = lane_masses();
    double incl = wave_incl_scan(ls, lane);
    double Z = __shfl(incl, kWave - 1, kWave);

    if (!(Z > 0.0) && D.mode) {
        // The residual vanished through rounding: draw from p alone with the
        // same uniform (a tile pass over the row, rare).
        D.mode = 0;
        for (int t = 0; t < ntiles; ++t) {
            const int j = t * kWave + lane;
            float xp[P], d[P];
            if (j < nvec)
                load_vec<E, ALIGNED>(prow, V, j, xp);
            else
#pragma unroll
                for (int e = 0; e < P; ++e) xp[e] = -__builtin_huge_valf();
            masses(xp, xp, D, d);
            const double tot = wave_sum(lane_total(d));
            if (lane == kWave - 1) tm[t] = tot;
        }
        __syncthreads();
        ls = lane_masses();
        incl = wave_incl_scan(ls, lane);
        Z = __shfl(incl, kWave - 1, kWave);
    }
    if (!(Z > 0.0)) {  // no finite logit in the row: nothing can be drawn
        if (lane == 0) *dst = -1;
        return;
    }
    const double target = Pm.u * Z;

    // 1. the lane whose tiles hold the crossing
    const double up = __shfl_up(incl, 1, kWave);
    const double excl = lane > 0 ? up : 0.0;
    uint64_t mk = ballot(ls > 0.0 && incl > target);
    const uint64_t pos_lanes_t = ballot(ls > 0.0);
    const int L = mk ? first_lane(mk) : (pos_lanes_t ? last_lane(pos_lanes_t) : -1);
    // 2. the tile, walked in order by that lane
    int tsel = -1;
    double trel = 0.0;
    if (L >= 0 && lane == L) {
        double run = excl, run_last = 0.0;
        int last = -1;
        for (int t = lt0; t < lt1; ++t) {
            const int k = t - lt0;
            double m = 0.0;
#pragma unroll
            for (int q = 0; q < kSelRegs; ++q) m = q == k ? tmr[q] : m;  // registers, not memory
            if (k >= kSelRegs) m = tm[t];
            if (m > 0.0) {
                if (run + m > target) {
                    tsel = t;
                    trel = target - run;
                    break;
                }
                last = t;
                run_last = run;
            }
            run += m;
        }
        if (tsel < 0) {
            tsel = last;
            trel = target - run_last;
        }
    }
    tsel = __shfl(tsel, L < 0 ? 0 : L, kWave);
    trel = __shfl(trel, L < 0 ? 0 : L, kWave);
    if (L < 0 || tsel < 0 || tsel >= ntiles) {  // unreachable for finite rows; never index with it
        if (lane == 0) *dst = -1;
        return;
    }

    // 3. the lane of that tile, then the element of that lane
    const int j = tsel * kWave + lane;
    float xp[P], xq[P], d[P];
    if (j < nvec) {
        load_vec<E, ALIGNED>(prow, V, j, xp);
        if (D.mode) {
            DraftStaged<E, EQ, ALIGNED> q;
            q.load(qrow, V, j);
            q.get(xq);
        } else
#pragma unroll
            for (int e = 0; e < P; ++e) xq[e] = -__builtin_huge_valf();
    } else {
#pragma unroll
        for (int e = 0; e < P; ++e) xp[e] = xq[e] = -__builtin_huge_valf();
    }
    masses(xp, xq, D, d);
    const double lm = lane_total(d);
    const double inc2 = wave_incl_scan(lm, lane);
    const double ex2 = __shfl_up(inc2, 1, kWave);
    mk = ballot(lm > 0.0 && inc2 > trel);
    const uint64_t pos_lanes = ballot(lm > 0.0);
    const int L2 = mk ? first_lane(mk) : (pos_lanes ? last_lane(pos_lanes) : -1);
    if (L2 < 0) {
        if (lane == 0) *dst = -1;
        return;
    }
    if (lane == L2) {
        double run = lane > 0 ? ex2 : 0.0;
        int pick = -1, last = -1;
#pragma unroll
        for (int e = 0; e < P; ++e) {
            run += static_cast<double>(d[e]);
            if (d[e] > 0.0f) {
                last = e;
                if (pick < 0 && run > trel) pick = e;
            }
        }
        if (pick < 0) pick = last;
        *dst = j * P + pick;
    }
}

// ---- dead-row skipping (stochastic chains without lse outputs) --------------------
//
// The protocol is described with SkipCtl.  Here the segments of position p are
// those of target row p and draft row p; its decision is the same fp64 merge,
// gather and ratio test as the full-read path.

__global__ __launch_bounds__(kBlock) void k_zero_words(uint32_t *__restrict__ p, long long n) {
    for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<long long>(gridDim.x) * blockDim.x)
        p[i] = 0;
}

// Words a wave hands to another without a ticket are marked so that a written
// word is never 0 (the words start at 0): a segment's R as its bits with the
// sign flipped (-0 taken as +0 first), its s >= 0 with the sign bit set, a
// row's log-sum like R.
__device__ __forceinline__ uint32_t mark_R(float R) {
    uint32_t u = __float_as_uint(R);
    if (u == 0x80000000u) u = 0u;
    return u ^ 0x80000000u;
}
__device__ __forceinline__ float unmark_R(uint32_t w) { return __uint_as_float(w ^ 0x80000000u); }
__device__ __forceinline__ float canonical_R(float R) { return unmark_R(mark_R(R)); }
__device__ __forceinline__ uint64_t mark_s(double s) {
    return static_cast<uint64_t>(__double_as_longlong(s)) | (1ull << 63);
}
__device__ __forceinline__ double unmark_s(uint64_t w) {
    return __longlong_as_double(static_cast<long long>(w & ~(1ull << 63)));
}
__device__ __forceinline__ uint64_t mark_L2(double v) {
    uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
    if (u == (1ull << 63)) u = 0;
    return u ^ (1ull << 63);
}
__device__ __forceinline__ double unmark_L2(uint64_t w) {
    return __longlong_as_double(static_cast<long long>(w ^ (1ull << 63)));
}

// The row merge over partials held one per lane, by the lanes where `member`.
__device__ __forceinline__ double merge_lanes(float R, double s, bool member) {
    const float Rm = wave_max(member ? R : -__builtin_huge_valf());
    double acc = 0.0;
    if (Rm != -__builtin_huge_valf() && member && s > 0.0)
        acc = s * exp2(static_cast<double>(R) - static_cast<double>(Rm));
    acc = wave_sum(acc);
    return acc > 0.0 ? static_cast<double>(Rm) + log2(acc) : -__builtin_huge_val();
}

// The row merge over marked words [base, base + segs), all written, except
// segment `own` (segs: none), which is this wave's (R, s).
__device__ __forceinline__ double merge_row_marked(uint32_t *wR, uint64_t *wS, long long base, int segs,
                                                   int own, float R, double s, int lane) {
    float Rm = -__builtin_huge_valf();
    for (int sg = lane; sg < segs; sg += kWave)
        Rm = fmaxf(Rm, sg == own ? canonical_R(R) : unmark_R(shared_load(&wR[base + sg])));
    Rm = wave_max(Rm);
    double acc = 0.0;
    if (Rm != -__builtin_huge_valf()) {
        for (int sg = lane; sg < segs; sg += kWave) {
            const double ss = sg == own ? s : unmark_s(shared_load(&wS[base + sg]));
            const float Rs = sg == own ? canonical_R(R) : unmark_R(shared_load(&wR[base + sg]));
            if (ss > 0.0) acc += ss * exp2(static_cast<double>(Rs) - static_cast<double>(Rm));
        }
    }
    acc = wave_sum(acc);
    return acc > 0.0 ? static_cast<double>(Rm) + log2(acc) : -__builtin_huge_val();
}

// Outputs of request b decided at n (mode 1: rejection at n, residual of
// rows n; mode 0: bonus from target row K), written by one wave that holds
// draft i and the draw uniform of position i in lane i (K <= 31).
__device__ __forceinline__ void skip_finish(int xl, float usl, int b, int K, int V, int n, int mode,
                                            double L2p, double L2q, int32_t *__restrict__ accept_len,
                                            int32_t *__restrict__ out_tokens,
                                            int32_t *__restrict__ status, ResidParam *__restrict__ rp,
                                            int lane) {
    bool bad = false;
    int32_t *tok = out_tokens + static_cast<long long>(b) * (K + 1);
    for (int i = lane; i <= K; i += kWave) {
        const int x = i < K ? xl : 0;
        if (i < K && (x < 0 || x >= V)) bad = true;
        tok[i] = i < n ? x : -1;
    }
    const bool any_bad = ballot(bad) != 0;
    const float u_n = __shfl(usl, n, kWave);
    if (lane == 0) {
        accept_len[b] = n;
        if (status) status[b] = any_bad ? 1 : 0;
        ResidParam P;
        P.pos = n;
        P.u = static_cast<double>(u_n);
        P.row_p = static_cast<long long>(b) * (K + 1) + n;
        P.L2p = L2p;
        P.mode = mode;
        P.row_q = mode ? static_cast<long long>(b) * K + n : 0;
        P.L2q = mode ? L2q : 0.0;
        draw_constants(P);
        rp[b] = P;
    }
}

template <typename E, bool ALIGNED, int U>
__global__ __launch_bounds__(kBlock) void k_skip_stats(
    const typename E::storage *__restrict__ tgt, const typename E::storage *__restrict__ drf,
    const int32_t *__restrict__ drafts, const float *__restrict__ ua, const float *__restrict__ us,
    int B, int K, int V, int nvec, int segs, double c, float c_hi, float c_lo, float *part_R,
    double *part_s, double *L2, SkipCtl ctl, int early, int rot, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ out_tokens, int32_t *__restrict__ status, ResidParam *__restrict__ rp) {
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned wave = skip_wave_index();
    const unsigned per_pos = static_cast<unsigned>(B) * 2u * static_cast<unsigned>(segs);
    if (wave >= per_pos * static_cast<unsigned>(K + 1)) return;
    const int p = static_cast<int>(wave / per_pos);
    const unsigned rem = wave - static_cast<unsigned>(p) * per_pos;
    const unsigned slot = rem / (2u * static_cast<unsigned>(segs));
    const int r = static_cast<int>(rem - slot * 2u * static_cast<unsigned>(segs));
    const int kind = r / segs, sg = r - kind * segs;
    const int b = skip_request(slot, p, B, rot);
    if (kind == 1 && p == K) return;  // no draft row at the bonus position
    // position 0's rows are always needed: no test, no wait before their loads
    if (p > 0 && (early ? skip_row_dead(ctl, b, p) : uniform(shared_load(&ctl.finished[b])) != 0)) return;

    const long long rows_t = static_cast<long long>(B) * (K + 1);
    const long long gt = static_cast<long long>(b) * (K + 1) + p;
    const long long gd = rows_t + static_cast<long long>(b) * K + p;
    const long long g = kind == 0 ? gt : gd;
    const typename E::storage *base = kind == 0 ? tgt + gt * static_cast<long long>(V)
                                                : drf + (static_cast<long long>(b) * K + p) * static_cast<long long>(V);
    int v0, v1;
    skip_segment(sg, nvec, segs, v0, v1);
    // the wave that will decide position p (the last of its partials, see
    // below) fetches the draft, the two logits it is scored with and its
    // uniform now, so that no load waits after the partials are in
    const bool decider = r == (p < K ? 2 : 1) * segs - 1;
    int xd = -1;
    float ud = 0.0f;
    // raw storage bits, read through readfirstlane only where they are used
    // (that keeps the wait for them there, not before the segment's loads)
    unsigned xp_raw = 0, xq_raw = 0;
    // and for the request's finish: draft i and the draw uniform of position
    // i in lane i (K <= 31)
    int xl = 0;
    float usl = 0.0f;
    if (decider) {
        if (lane < K) xl = drafts[static_cast<long long>(b) * K + lane];
        if (lane <= K) usl = us[static_cast<long long>(b) * (K + 1) + lane];
    }
    if (decider && p < K) {
        xd = uniform(drafts[static_cast<long long>(b) * K + p]);
        ud = ua[static_cast<long long>(b) * K + p];
        if (xd >= 0 && xd < V) {
            xp_raw = storage_bits(tgt[gt * V + xd]);
            xq_raw = storage_bits(drf[(static_cast<long long>(b) * K + p) * V + xd]);
        }
    }
    float R;
    double sum;
    segment_stats_chunked<E, ALIGNED, U, kSkipChunks>(base, V, v0, v1, c_hi, c_lo, lane, R, sum);
    const int nrows = 2 * K + 1;
    double *L2b = L2 + static_cast<long long>(b) * nrows;
    // Every wave but the last of (b, p) leaves its partial as two marked words
    // (never 0; they start at 0) and goes.  The last one, the draft row's last
    // segment (the target row's at the bonus position), is dispatched after
    // the others: it collects their partials, or learns from the same test
    // they made that they skipped theirs and the request is settled.
    uint32_t *wR = reinterpret_cast<uint32_t *>(part_R);
    uint64_t *wS = reinterpret_cast<uint64_t *>(part_s);
    const int nparts = (p < K ? 2 : 1) * segs, mine = nparts - 1;
    if (r != mine) {
        if (lane == 0) {
            shared_store(&wR[g * segs + sg], mark_R(R));
            shared_store(&wS[g * segs + sg], mark_s(sum));
        }
        return;
    }
    // partial i of (b, p): segment i % segs of the target row (i < segs) or of
    // the draft row
    auto part_index = [&](int i) { return i < segs ? gt * segs + i : gd * segs + (i - segs); };
    float Ri = -__builtin_huge_valf();
    double si = 0.0;
    bool complete = false;
    for (int t = 0; t < kSkipPollCap; ++t) {
        bool missing = false;
        for (int i = lane; i < mine; i += kWave) {
            const uint32_t a = shared_load(&wR[part_index(i)]);
            const uint64_t s2 = shared_load(&wS[part_index(i)]);
            missing |= a == 0 || s2 == 0;
            if (i == lane) {
                Ri = unmark_R(a);
                si = unmark_s(s2);
            }
        }
        if (ballot(missing) == 0) {
            complete = true;
            break;
        }
        if (early ? skip_row_dead(ctl, b, p) : uniform(shared_load(&ctl.finished[b])) != 0) return;
        __builtin_amdgcn_s_sleep(2);
    }
    if (!complete) return;  // never decide on part of a row
    if (lane == mine) {
        Ri = canonical_R(R);
        si = sum;
    }
    double L2p, L2q = 0.0;
    if (nparts <= kWave) {  // every partial is held by the lane of its index
        const bool tl = lane < segs, dl = lane >= segs && lane < nparts;
        L2p = merge_lanes(Ri, si, tl);
        if (p < K) L2q = merge_lanes(Ri, si, dl);
    } else {
        L2p = merge_row_marked(wR, wS, gt * segs, segs, p < K ? segs : segs - 1, R, sum, lane);
        if (p < K) L2q = merge_row_marked(wR, wS, gd * segs, segs, segs - 1, R, sum, lane);
    }
    uint64_t bits = 1ull << p;
    if (p < K) {
        double ratio = 0.0;
        if (xd >= 0 && xd < V) {
            const double px = exp2(static_cast<double>(from_bits<E>(uniform(xp_raw))) * c - L2p);
            const double qx = exp2(static_cast<double>(from_bits<E>(uniform(xq_raw))) * c - L2q);
            ratio = qx == 0.0 ? __builtin_huge_val() : px / qx;
        }
        if (!(static_cast<double>(ud) < ratio)) bits |= 1ull << (32 + p);
    }
    // The decision is one atomic OR; the wave whose OR completes the request's
    // decided prefix finishes it.  The log-sums of a decided position are
    // marked words too and need not land before its OR: the finisher polls for
    // those of the position it draws from.
    uint64_t *wL = reinterpret_cast<uint64_t *>(L2b);
    uint64_t old = 0;
    if (lane == 0) {
        if (p < K) shared_store(&wL[K + 1 + p], mark_L2(L2q));
        shared_store(&wL[p], mark_L2(L2p));
        old = __hip_atomic_fetch_or(&ctl.mask[b], bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    old = uniform(static_cast<uint64_t>(__shfl(static_cast<long long>(old), 0, kWave)));
    if (skip_prefix(old, K) >= 0) return;  // the request was complete already
    const int n = skip_prefix(old | bits, K);
    if (n < 0) return;
    double L2pn = L2p, L2qn = L2q;
    if (n != p) {
        uint64_t w = 0;
        if (lane < (n < K ? 2 : 1)) {
            uint64_t *q = &wL[lane == 0 ? n : K + 1 + n];
            for (int t = 0; t < kSkipPollCap && (w = shared_load(q)) == 0; ++t) __builtin_amdgcn_s_sleep(1);
        }
        const long long w0 = __shfl(static_cast<long long>(w), 0, kWave);
        const long long w1 = __shfl(static_cast<long long>(w), 1, kWave);
        L2pn = unmark_L2(static_cast<uint64_t>(w0));
        L2qn = n < K ? unmark_L2(static_cast<uint64_t>(w1)) : 0.0;
    }
    skip_finish(xl, usl, b, K, V, n, n < K ? 1 : 0, L2pn, L2qn, accept_len, out_tokens, status, rp, lane);
    skip_finished(ctl, b, lane);
}

template <typename E, bool ALIGNED>
hipError_t skip_stats_t(const void *tgt, const void *drf, const int32_t *drafts, const float *ua,
                        const float *us, int B, int K, int V, const RowGeom &g, const Scale &sc,
                        float *part_R, double *part_s, double *L2, const SkipCtl &ctl,
                        int32_t *accept_len, int32_t *out_tokens, int32_t *status, ResidParam *rp,
                        hipStream_t s) {
    using T = typename E::storage;
    const long long nwaves = static_cast<long long>(K + 1) * B * 2 * g.segs;
    const long long blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    const bool early = skip_early(B, 2, V, sizeof(T));
    return launch_kernel(k_skip_stats<E, ALIGNED, kSkipVecsPerLane>, dim3(static_cast<unsigned>(blocks)),
                         dim3(kBlock), 0, s, static_cast<const T *>(tgt), static_cast<const T *>(drf),
                         drafts, ua, us, B, K, V, g.nvec, g.segs, sc.c, sc.c_hi, sc.c_lo, part_R, part_s,
                         L2, ctl, static_cast<int>(early), skip_rotation(B, early), accept_len, out_tokens, status,
                         rp);
}

template <typename E, bool ALIGNED>
hipError_t rowstats_t(const void *tgt, const void *drf, long long rows_t, long long rows_total, int V,
                      const RowGeom &g, const Scale &sc, float *part_R, double *part_s,
                      hipStream_t s) {
    using T = typename E::storage;
    const long long nwaves = rows_total * g.segs;
    const long long blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    return launch_kernel(k_rowstats<E, ALIGNED, kStatsVecsPerLane>, dim3(static_cast<unsigned>(blocks)),
                         dim3(kBlock), 0, s, static_cast<const T *>(tgt), static_cast<const T *>(drf),
                         rows_t, nwaves, V, g.nvec, g.segs, sc.c_hi, sc.c_lo, part_R, part_s);
}

}  // namespace

hipError_t launch_rowstats(const void *tgt, const void *drf, long long rows_t, long long rows_total,
                           int V, const RowGeom &g, sv_dtype dt, const Scale &sc, float *part_R,
                           double *part_s, hipStream_t s) {
    if (dt == SV_BF16)
        return g.aligned ? rowstats_t<BF16, true>(tgt, drf, rows_t, rows_total, V, g, sc, part_R, part_s, s)
                         : rowstats_t<BF16, false>(tgt, drf, rows_t, rows_total, V, g, sc, part_R, part_s, s);
    return g.aligned ? rowstats_t<F32, true>(tgt, drf, rows_t, rows_total, V, g, sc, part_R, part_s, s)
                     : rowstats_t<F32, false>(tgt, drf, rows_t, rows_total, V, g, sc, part_R, part_s, s);
}

bool skip_supported(int K) { return K <= kSkipMaxK; }

size_t skip_ctl_bytes(int B, int) { return sizeof(uint64_t) * B + sizeof(unsigned) * static_cast<size_t>(B); }

hipError_t clear_words(void *base, size_t bytes, hipStream_t s) {
    const long long words = static_cast<long long>(bytes / sizeof(uint32_t));
    const long long zb = std::max<long long>(1, std::min<long long>(1024, (words + kBlock - 1) / kBlock));
    trace_select(-1);  // the clearing launch is not traced
    hipLaunchKernelGGL(k_zero_words, dim3(static_cast<unsigned>(zb)), dim3(kBlock), 0, s,
                       reinterpret_cast<uint32_t *>(base), words);
    return hipGetLastError();
}

void skip_ctl_carve(void *base, int B, int, SkipCtl *ctl) {
    ctl->mask = static_cast<uint64_t *>(base);
    ctl->finished = reinterpret_cast<unsigned *>(ctl->mask + B);
    ctl->lim = ctl->finished + B;  // past skip_ctl_bytes: only the greedy chain's words hold it
}

hipError_t launch_skip(const void *tgt, const void *drf, const int32_t *drafts, const float *ua,
                       const float *us, int B, int K, int V, const RowGeom &g, sv_dtype dt,
                       const Scale &sc, float *part_R, double *part_s, double *L2, void *ctl_base,
                       int32_t *accept_len, int32_t *out_tokens, int32_t *status, ResidParam *rp,
                       hipStream_t s) {
    SkipCtl ctl;
    // the partials, the log-sums and the control words are marked words that
    // start at 0; the workspace holds them in that order, back to back
    skip_ctl_carve(ctl_base, B, K, &ctl);
    char *first = reinterpret_cast<char *>(part_R);
    char *end = static_cast<char *>(ctl_base) + skip_ctl_bytes(B, K);
    if (first > reinterpret_cast<char *>(part_s) || reinterpret_cast<char *>(part_s) > reinterpret_cast<char *>(L2) ||
        reinterpret_cast<char *>(L2) > static_cast<char *>(ctl_base))
        return hipErrorInvalidValue;
    hipError_t e = clear_words(first, static_cast<size_t>(end - first), s);
    if (e != hipSuccess) return e;
    trace_select(SV_K_SKIP_STATS);
#define SV_SK(E, A) skip_stats_t<E, A>(tgt, drf, drafts, ua, us, B, K, V, g, sc, part_R, part_s, L2, ctl, accept_len, out_tokens, status, rp, s)
    if (dt == SV_BF16) return g.aligned ? SV_SK(BF16, true) : SV_SK(BF16, false);
    return g.aligned ? SV_SK(F32, true) : SV_SK(F32, false);
#undef SV_SK
}

hipError_t launch_accept(const void *tgt, const void *drf, const int32_t *drafts, const float *ua,
                         const float *us, int B, int K, int V, sv_dtype dt, const Scale &sc,
                         const PartRows &pt, const PartRows &pd, const float *xlog, double *L2,
                         int32_t *accept_len, int32_t *out_tokens, float *lse_t, float *lse_d,
                         int32_t *status, ResidParam *rp, hipStream_t s) {
    const int nrows = 2 * K + 1;
    const size_t per_row = static_cast<size_t>(pt.segs) * (sizeof(float) + sizeof(double));
    const int lr = (K > 0 && pd.segs != pt.segs) || per_row > static_cast<size_t>(kMergeLdsBytes)
                       ? 0
                       : static_cast<int>(std::min<size_t>(nrows, kMergeLdsBytes / per_row));
    const size_t lds = sizeof(double) * static_cast<size_t>(nrows) + static_cast<size_t>(lr) * per_row;
#define SV_ACC(E, FUSED)                                                                                  \
    launch_kernel(k_accept<E, FUSED>, dim3(B), dim3(kBlock), lds, s,                                       \
                  static_cast<const typename E::storage *>(tgt), static_cast<const typename E::storage *>(drf), \
                  drafts, ua, us, B, K, V, pt, pd, lr, sc.c, xlog, L2, accept_len, out_tokens, lse_t, lse_d, \
                  status, rp)
    if (dt == SV_BF16) return xlog ? SV_ACC(BF16, true) : SV_ACC(BF16, false);
    return xlog ? SV_ACC(F32, true) : SV_ACC(F32, false);
#undef SV_ACC
}

namespace {
template <typename E, typename EQ, bool ALIGNED>
hipError_t resid_mass_t(const void *tgt, const void *drf, int B, int V, const RowGeom &g,
                        const Scale &sc, const ResidParam *rp, double *tile_mass, hipStream_t s) {
    const int tpw = resid_tiles_per_wave(B, g.ntiles);
    const int wpr = (g.ntiles + tpw - 1) / tpw;
    const long long nwaves = static_cast<long long>(B) * wpr;
    const long long blocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    return launch_kernel(k_resid_mass<E, EQ, ALIGNED, kResidGroup>, dim3(static_cast<unsigned>(blocks)),
                         dim3(kBlock), 0, s, static_cast<const typename E::storage *>(tgt),
                         static_cast<const typename EQ::storage *>(drf), B, V, g.nvec, g.ntiles, wpr, tpw,
                         sc.c_hi, sc.c_lo, rp, tile_mass);
}
template <typename E, typename EQ, bool ALIGNED>
hipError_t resid_select_t(const void *tgt, const void *drf, int B, int K, int V, const RowGeom &g,
                          const Scale &sc, const ResidParam *rp, double *tile_mass,
                          int32_t *out_tokens, hipStream_t s) {
    return launch_kernel(k_resid_select<E, EQ, ALIGNED>, dim3(B), dim3(kWave), 0, s,
                         static_cast<const typename E::storage *>(tgt),
                         static_cast<const typename EQ::storage *>(drf), B, K, V, g.nvec, g.ntiles, sc.c_hi,
                         sc.c_lo, rp, tile_mass, out_tokens);
}

// The three pairings the draw reads: both rows bf16, both fp32, or fp32
// target rows beside bf16 draft rows (the fused LM-head form).  The aligned
// form needs g.aligned (the target rows) and the draft rows aligned to their
// own vector: 16 bytes, or 8 for bf16 beside fp32 (V % 4 == 0 is part of
// g.aligned, so every draft row then starts on that boundary too).
template <typename F>
hipError_t resid_dispatch(sv_dtype dt, sv_dtype dq, const RowGeom &g, const void *drf, F &&f) {
    const uintptr_t q = reinterpret_cast<uintptr_t>(drf);
    if (dt == SV_BF16 && dq == SV_BF16) {
        const bool al = g.aligned && (q & 15u) == 0;
        return al ? f(BF16{}, BF16{}, std::true_type{}) : f(BF16{}, BF16{}, std::false_type{});
    }
    if (dt == SV_F32 && dq == SV_F32) {
        const bool al = g.aligned && (q & 15u) == 0;
        return al ? f(F32{}, F32{}, std::true_type{}) : f(F32{}, F32{}, std::false_type{});
    }
    if (dt == SV_F32 && dq == SV_BF16) {
        const bool al = g.aligned && (q & 7u) == 0;
        return al ? f(F32{}, BF16{}, std::true_type{}) : f(F32{}, BF16{}, std::false_type{});
    }
    return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_merge_parts(const float *R, const double *S, long long rows, int segs, float *outR,
                              double *outS, hipStream_t s) {
    const long long blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    return launch_kernel(k_merge_parts, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, R, S, rows, segs,
                         outR, outS);
}

hipError_t launch_resid_mass(const void *tgt, const void *drf, int B, int V, const RowGeom &g,
                             sv_dtype dt, sv_dtype dq, const Scale &sc, const ResidParam *rp,
                             double *tile_mass, hipStream_t s) {
    return resid_dispatch(dt, dq, g, drf, [&](auto e, auto eq, auto al) {
        return resid_mass_t<decltype(e), decltype(eq), decltype(al)::value>(tgt, drf, B, V, g, sc, rp,
                                                                              tile_mass, s);
    });
}

hipError_t launch_resid_select(const void *tgt, const void *drf, int B, int K, int V,
                               const RowGeom &g, sv_dtype dt, sv_dtype dq, const Scale &sc,
                               const ResidParam *rp, double *tile_mass, int32_t *out_tokens,
                               hipStream_t s) {
    return resid_dispatch(dt, dq, g, drf, [&](auto e, auto eq, auto al) {
        return resid_select_t<decltype(e), decltype(eq), decltype(al)::value>(tgt, drf, B, K, V, g, sc, rp,
                                                                                tile_mass, out_tokens, s);
    });
}

}  // namespace sv
