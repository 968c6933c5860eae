// sv_lmhead.hip -- the target's LM-head projection fused with what verification
// needs of its rows: logits = H W^T are formed tile by tile on the matrix cores
// and reduced at once, per row and 128-column segment, to
//   - (max, lowest index) keys, for greedy verification (k_lmhead<kEpiArgmax>);
//   - (R, s) statistics in the form the streaming row-statistics pass makes
//     (R = fp32(max * c_hi), s = sum 2^(x c - R)), plus the logit at the row's
//     draft token, for speculative sampling (k_lmhead<kEpiStats>);
// so the logits are never written.  The one row per request a sampled token is
// drawn from is formed again afterwards and written (k_lmhead<kEpiRows>, its H
// rows picked by the acceptance kernel's result).
//
// What it feeds: the speculative-decoding tutorial page, section
// "一轮推测解码究竟发生什么" (the target scores all gamma+1 positions in one
// parallel pass; greedy verification keeps drafts while they equal the target's
// argmax), and the DLite notes, section 2 (the D x V vocabulary projection is
// the cost a drafter avoids repeating per position).
//
// k_lmhead: C[m][n] = sum_k H[m][k] W[n][k] with H [M][D] and W [V][D]
// bf16, both k-contiguous.  A workgroup of 8 waves (two per SIMD) owns a
// 256 x 256 tile of C and walks D in steps of 64, each computed as four
// 16-deep quarters.  The H and W slabs of a step go straight from global
// memory into LDS (global_load_lds, 16 bytes per lane, no registers); a slab
// row is one whole 128-byte cache line, which the L2 serves at about twice the
// rate of half lines.  LDS holds two H slots and three W slots (160 KB): H is
// loaded two steps ahead and W, which misses to HBM more often, three.  The
// eight 16-byte chunks of row r are stored in the order c ^ ((r >> 1) & 7), so
// the fragment reads of 16 consecutive rows hit distinct banks.  Each wave
// holds a 64 x 128 part as 2 x 4 tiles of v_mfma_f32_32x32x16_bf16
// accumulators (fp32).
//
// Schedule of step s, quarters q0..q3, fragments double-buffered:
//   q0: read q1's fragments; wait for q0's; MFMAs of q0
//   q1: read q2's; wait for q1's; MFMAs of q1
//   q2: read q3's; wait for q2's; wait for this wave's loads of step s + 1;
//       barrier; MFMAs of q2
//   q3: read q0's of step s + 1; wait for q3's; barrier (every wave is done
//       with step s's slots); loads of H(s + 2) and W(s + 3) into them;
//       MFMAs of q3
// The fragment reads of one quarter are always in flight under the MFMAs of
// the previous one, across the barriers too.  They are issued as inline
// ds_read instructions with explicit lgkmcnt waits tied to the fragment
// registers: with LDS DMA in flight the compiler would otherwise wait for
// every LDS read before each group of MFMAs.
//
// Workgroups are numbered so that the row tiles of one column tile run
// together on one XCD (consecutive workgroup ids go to consecutive XCDs): the
// column tile's W slab is then read from HBM once and shared through that
// XCD's L2.
#include <limits.h>

#include <type_traits>

#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define SV_LDS __attribute__((address_space(3)))

constexpr int kXcds = 8;
constexpr int kTM = 256, kTN = 256, kTK = 64;  // workgroup tile and D step
constexpr int kRowB = kTK * 2;                 // LDS bytes per slab row (one cache line)
constexpr int kChunks = kRowB / 16;            // 16-byte chunks per slab row (8)
constexpr int kSlab = kTM * kRowB;             // bytes of one operand slab (32 KB)
constexpr int kHSlots = 2, kWSlots = 3;        // H loaded 2 steps ahead, W 3
constexpr int kSegCols = 128;                  // columns per argmax key (one wave's width)
constexpr int kLmWaves = 8;
constexpr int kLmThreads = kLmWaves * kWave;
constexpr int kTileRows = 32;                  // rows (and columns) of one MFMA tile
constexpr int kDmaPerOperand = kSlab / 1024 / kLmWaves;  // 1 KB DMA instructions per wave (4)
constexpr int kEpiRowB = 272;                  // epilogue: bytes per tile row (32 x 8 + 16 of padding)
constexpr int kEpiWaveB = 64 * kEpiRowB + 64 * 4;  // a wave's epilogue area: 64 rows + one float per row
static_assert(kLmWaves * kEpiWaveB <= (kHSlots + kWSlots) * kSlab, "epilogue areas fit in the ring");

// H slots first, then W slots
__shared__ __align__(1024) char ring[(kHSlots + kWSlots) * kSlab];

template <int N> using IC = std::integral_constant<int, N>;

// vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One 16-byte fragment read at LDS byte address addr + OFF.  The result is not
// valid until an lgkmcnt wait that names it (LDS_WAIT below).
template <int OFF> __device__ __forceinline__ bf16x8 lds_read(uint32_t addr, IC<OFF>) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
    bf16x8 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

// Wait until at most 6 LDS reads are outstanding (the six issued after the
// named fragments), and make the named fragments depend on that wait.
#define LDS_WAIT6(a0, a1, b0, b1, b2, b3) \
    asm volatile("s_waitcnt lgkmcnt(6)" : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3))
#define LDS_WAIT0(a0, a1, b0, b1, b2, b3) \
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3))
#define SV_BARRIER() asm volatile("s_barrier" ::: "memory")

// What the epilogue makes of a finished tile.
enum LmEpi { kEpiArgmax = 0, kEpiStats = 1, kEpiRows = 2 };
struct LmOut {
    int segs;               // 128-column segments per row
    uint64_t *keys;         // argmax: [M][segs] keys
    float *part_R;          // stats: [M][segs] R
    double *part_s;         // stats: [M][segs] s
    float *xlog;            // stats: [M] the logit at each row's draft token
    const int32_t *drafts;  // stats: [M / (K+1)][K] draft ids (row i of a request scores draft i)
    int K;
    float c_hi, c_lo;       // stats: log2(e)/T split in two floats
    float *rows;            // rows: [M][V] fp32 logits
    const ResidParam *rp;   // rows: output row m projects H row m (K+1) + rp[m].pos
};

template <int EPI>
__global__ __launch_bounds__(kLmThreads, 1) void k_lmhead(const uint4 *__restrict__ H,
                                                      const uint4 *__restrict__ W, int M, int D, int V,
                                                      int mtiles, int ntiles, LmOut o) {
    const int bid = blockIdx.x;
    const int xcd = bid % kXcds, j = bid / kXcds;
    const int mt = j % mtiles;
    const int nt = (j / mtiles) * kXcds + xcd;
    if (nt >= ntiles) return;
    const int m0 = mt * kTM, n0 = nt * kTN;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int dv = D / 8;  // 16-byte chunks per row

    // DMA mapping: instruction i of wave w fills slab rows 8 q .. 8 q + 7 for
    // q = 8 i + w; lane l writes 16 bytes at 16 l, i.e. row 8 q + l / 8,
    // stored chunk l % 8, which holds the row's logical chunk
    // (l % 8) ^ ((row >> 1) & 7) (the swizzle is an involution).  Offsets are
    // 32-bit 16-byte-chunk counts; rows past M or V read the last row.  For
    // kEpiRows, tile row m is H row m (K + 1) + rp[m].pos.
    auto hrow = [&](int m) {
        if constexpr (EPI == kEpiRows)
            return m * (o.K + 1) + o.rp[m].pos;
        else
            return m;
    };
    int ga0, ga1, ga2, ga3, gb0, gb1, gb2, gb3;
#define SV_GOFF(i, GA, GB)                                        \
    {                                                             \
        const int r = 8 * (kLmWaves * (i) + w) + lane / kChunks;  \
        const int c = (lane % kChunks) ^ ((r >> 1) & 7);          \
        GA = hrow(min(m0 + r, M - 1)) * dv + c;                   \
        GB = min(n0 + r, V - 1) * dv + c;                         \
    }
    SV_GOFF(0, ga0, gb0)
    SV_GOFF(1, ga1, gb1)
    SV_GOFF(2, ga2, gb2)
    SV_GOFF(3, ga3, gb3)
#undef SV_GOFF
    static_assert(kDmaPerOperand == 4, "four DMA instructions per operand per wave");
    const int nk = D / kTK;
    // kEpiStats: the draft token scored by row m0 + wm 64 + lane (-1 if none),
    // fetched now so the epilogue never waits on a load
    int xdraft = -1;
    if constexpr (EPI == kEpiStats) {
        const int row = m0 + wm * 64 + lane;
        const int req = row / (o.K + 1), i = row - req * (o.K + 1);
        if (row < M && i < o.K) xdraft = o.drafts[static_cast<long long>(req) * o.K + i];
    }
#define SV_ISSUE(SRC, G0, G1, G2, G3, slab, step)                                                    \
    {                                                                                                \
        const int k0 = (step) * kChunks;                                                             \
        char *sl = ring + (slab) * kSlab;                                                            \
        __builtin_amdgcn_global_load_lds(SRC + G0 + k0, (SV_LDS void *)(sl + (0 + w) * 1024), 16, 0, 0);  \
        __builtin_amdgcn_global_load_lds(SRC + G1 + k0, (SV_LDS void *)(sl + (8 + w) * 1024), 16, 0, 0);  \
        __builtin_amdgcn_global_load_lds(SRC + G2 + k0, (SV_LDS void *)(sl + (16 + w) * 1024), 16, 0, 0); \
        __builtin_amdgcn_global_load_lds(SRC + G3 + k0, (SV_LDS void *)(sl + (24 + w) * 1024), 16, 0, 0); \
    }
#define SV_ISSUE_H(slot, step) SV_ISSUE(H, ga0, ga1, ga2, ga3, (slot), step)
#define SV_ISSUE_W(slot, step) SV_ISSUE(W, gb0, gb1, gb2, gb3, kHSlots + (slot), step)

    // Fragment addresses per quarter q: lane l reads the 8 k-values of row
    // (l % 32) of a tile at logical chunk 2 q + l / 32, stored at that
    // ^ (((l % 32) >> 1) & 7) (tile rows are multiples of 32, so the swizzle
    // depends on the lane only).  Tile t of a slab sits 32 t rows further (an
    // immediate offset); the slot's byte offset is added per read group.
    const uint32_t lbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SV_LDS char *)ring));
    const int sw = ((lane & 31) >> 1) & 7;
    const uint32_t rowA = lbase + (wm * 64 + (lane & 31)) * kRowB;
    const uint32_t rowB = lbase + kHSlots * kSlab + (wn * 128 + (lane & 31)) * kRowB;
#define SV_CH(q) ((((2 * (q)) + (lane >> 5)) ^ sw) << 4)
    const uint32_t a0 = rowA + SV_CH(0), a1 = rowA + SV_CH(1), a2 = rowA + SV_CH(2), a3 = rowA + SV_CH(3);
    const uint32_t b0 = rowB + SV_CH(0), b1 = rowB + SV_CH(1), b2 = rowB + SV_CH(2), b3 = rowB + SV_CH(3);
#undef SV_CH

    f32x16 c00{}, c01{}, c02{}, c03{}, c10{}, c11{}, c12{}, c13{};
    bf16x8 p0, p1, q0, q1, q2, q3;  // fragments of one quarter (A tiles 0-1, B tiles 0-3)
    bf16x8 r0, r1, t0, t1, t2, t3;  // fragments of the next
#define SV_READ(AB, BB, A0, A1, B0, B1, B2, B3)                    \
    {                                                              \
        const uint32_t ab = (AB), bb = (BB);                       \
        A0 = lds_read(ab, IC<0>{});                                \
        A1 = lds_read(ab, IC<1 * kTileRows * kRowB>{});            \
        B0 = lds_read(bb, IC<0>{});                                \
        B1 = lds_read(bb, IC<1 * kTileRows * kRowB>{});            \
        B2 = lds_read(bb, IC<2 * kTileRows * kRowB>{});            \
        B3 = lds_read(bb, IC<3 * kTileRows * kRowB>{});            \
    }
#define SV_MFMA(A0, A1, B0, B1, B2, B3)                                          \
    c00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B0, c00, 0, 0, 0);        \
    c01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B1, c01, 0, 0, 0);        \
    c02 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B2, c02, 0, 0, 0);        \
    c03 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, B3, c03, 0, 0, 0);        \
    c10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B0, c10, 0, 0, 0);        \
    c11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B1, c11, 0, 0, 0);        \
    c12 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B2, c12, 0, 0, 0);        \
    c13 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B3, c13, 0, 0, 0);

    // prologue, in the order the steady state keeps (H(s + 2) then W(s + 3) per step)
    SV_ISSUE_W(0, 0)
    SV_ISSUE_H(0, 0)
    SV_ISSUE_W(1, min(1, nk - 1))
    SV_ISSUE_H(1, min(1, nk - 1))
    SV_ISSUE_W(2, min(2, nk - 1))
    wait_vm<3 * kDmaPerOperand>();  // this wave's W(0) and H(0) are in
    SV_BARRIER();                   // and every wave's
    uint32_t ho = 0, wo = 0;        // byte offsets of step s's H and W slots
    int hs = 0, ws = 0;             // their slot numbers
    SV_READ(a0 + ho, b0 + wo, p0, p1, q0, q1, q2, q3)
    // past the end, the last step is loaded again into slots nobody reads, and
    // the first quarter's reads of the step after the last are discarded
    for (int s = 0; s < nk; ++s) {
        const int hs_n = hs ^ 1, ws_n = ws == kWSlots - 1 ? 0 : ws + 1;
        const uint32_t ho_n = static_cast<uint32_t>(hs_n * kSlab), wo_n = static_cast<uint32_t>(ws_n * kSlab);
        SV_READ(a1 + ho, b1 + wo, r0, r1, t0, t1, t2, t3)
        LDS_WAIT6(p0, p1, q0, q1, q2, q3);
        SV_MFMA(p0, p1, q0, q1, q2, q3)
        SV_READ(a2 + ho, b2 + wo, p0, p1, q0, q1, q2, q3)
        LDS_WAIT6(r0, r1, t0, t1, t2, t3);
        SV_MFMA(r0, r1, t0, t1, t2, t3)
        SV_READ(a3 + ho, b3 + wo, r0, r1, t0, t1, t2, t3)
        LDS_WAIT6(p0, p1, q0, q1, q2, q3);
        // this wave's H(s + 1) and W(s + 1) are in: only W(s + 2), issued
        // after them, may still be outstanding
        wait_vm<kDmaPerOperand>();
        SV_BARRIER();
        SV_MFMA(p0, p1, q0, q1, q2, q3)
        SV_READ(a0 + ho_n, b0 + wo_n, p0, p1, q0, q1, q2, q3)
        LDS_WAIT6(r0, r1, t0, t1, t2, t3);
        SV_BARRIER();  // every wave is done with step s's slots
        SV_ISSUE_H(hs, min(s + 2, nk - 1))
        SV_ISSUE_W(ws, min(s + 3, nk - 1))
        SV_MFMA(r0, r1, t0, t1, t2, t3)
        hs = hs_n;
        ws = ws_n;
        ho = ho_n;
        wo = wo_n;
    }
#undef SV_MFMA
#undef SV_READ
#undef SV_ISSUE_W
#undef SV_ISSUE_H
#undef SV_ISSUE
    LDS_WAIT0(p0, p1, q0, q1, q2, q3);  // no LDS read still in flight
    wait_vm<0>();                       // no DMA may still target LDS when the workgroup ends

    // epilogue over this wave's 64 x 128 part: lanes l and l + 32 hold rows 4
    // apart, and lane l % 32 holds columns cb + l % 32 + 32 b, b = 0..3
    const int cb = n0 + wn * 128;
    const int lc = lane & 31;
    const f32x16 acc[2][4] = {{c00, c01, c02, c03}, {c10, c11, c12, c13}};
    const float ninf = -__builtin_huge_valf();
    if constexpr (EPI == kEpiRows) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + a * kTileRows + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= M) continue;
                float *dst = o.rows + static_cast<long long>(row) * V;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int col = cb + b * kTileRows + lc;
                    if (col < V) dst[col] = acc[a][b][r];
                }
            }
        }
        return;
    }
    // The row reductions go through LDS, free once every wave is done with
    // the ring: each lane reduces its own four columns of each of its 32
    // rows and leaves the partial in its wave's area (one 272-byte row per
    // tile row: 32 partials of up to 8 bytes, padded so that 16 lanes reading
    // 16 bytes each from 16 rows hit distinct banks); then lane j reduces row
    // j's 32 partials with 16 independent reads.  Cross-lane shuffle chains,
    // 32 of them per wave, would leave the CU idle for their latency instead.
    SV_BARRIER();
    const int seg = cb / kSegCols;
    if (seg >= o.segs) return;
    char *area = ring + w * kEpiWaveB;
    const int row_j = m0 + wm * 64 + lane;  // the row this lane reduces
#define SV_RL(a, r) ((a) * kTileRows + 8 * ((r) >> 2) + 4 * (lane >> 5) + ((r) & 3))
    if constexpr (EPI == kEpiArgmax) {
        // each lane's first maximum over its four columns, as a 64-bit key
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float best = ninf;
                int bi = INT_MAX;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int col = cb + lc + b * kTileRows;
                    const float x = col < V ? acc[a][b][r] : ninf;
                    if (x > best || (bi == INT_MAX && col < V)) {
                        best = x;
                        bi = col;
                    }
                }
                *reinterpret_cast<uint64_t *>(area + SV_RL(a, r) * kEpiRowB + lc * 8) = argmax_key(best, bi);
            }
        }
        asm volatile("" ::: "memory");
        const uint4 *kp = reinterpret_cast<const uint4 *>(area + lane * kEpiRowB);
        uint64_t mk = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const uint4 v = kp[q];
            const uint64_t k0 = static_cast<uint64_t>(v.x) | (static_cast<uint64_t>(v.y) << 32);
            const uint64_t k1 = static_cast<uint64_t>(v.z) | (static_cast<uint64_t>(v.w) << 32);
            mk = k0 > mk ? k0 : mk;
            mk = k1 > mk ? k1 : mk;
        }
        if (row_j < M) o.keys[static_cast<long long>(row_j) * o.segs + seg] = mk;
    } else {
        // (R, s) as the streaming pass forms them: R = fp32(max * c_hi) over
        // the 128 columns; each lane's four terms summed pairwise in fp32,
        // the 32 lanes in fp64 in lane order
        float *Rrow = reinterpret_cast<float *>(area + 64 * kEpiRowB);
        bool valid[4];  // this lane's columns inside the vocabulary
#pragma unroll
        for (int b = 0; b < 4; ++b) valid[b] = cb + lc + b * kTileRows < V;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float m = ninf;
#pragma unroll
                for (int b = 0; b < 4; ++b) m = fmaxf(m, valid[b] ? acc[a][b][r] : ninf);
                *reinterpret_cast<float *>(area + SV_RL(a, r) * kEpiRowB + lc * 4) = m;
            }
        }
        asm volatile("" ::: "memory");
        float mrow = ninf;
        {
            const float4 *fp = reinterpret_cast<const float4 *>(area + lane * kEpiRowB);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 v = fp[q];
                mrow = fmaxf(fmaxf(mrow, fmaxf(v.x, v.y)), fmaxf(v.z, v.w));
            }
        }
        const float Rj = mrow == ninf ? 0.0f : mrow * o.c_hi;  // all -inf: every term is 0
        Rrow[lane] = Rj;
        asm volatile("" ::: "memory");
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = SV_RL(a, r);
                const float R = Rrow[rl];
                float x[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float t = fast_exp2(fmaf(acc[a][b][r], o.c_lo, fmaf(acc[a][b][r], o.c_hi, -R)));
                    x[b] = valid[b] ? t : 0.0f;
                }
                *reinterpret_cast<double *>(area + rl * kEpiRowB + lc * 8) = static_cast<double>(pairwise_sum(x));
                // the logit at this row's draft, if it falls in this wave's columns
                const int row = m0 + wm * 64 + rl;
                const int xt = __shfl(xdraft, rl, kWave);
                const int rel = xt - cb;
                if (row < M && rel >= 0 && rel < 128 && xt < V && lc == (rel & 31)) {
                    const int bb = rel >> 5;
                    o.xlog[row] = bb == 0 ? acc[a][0][r] : bb == 1 ? acc[a][1][r]
                                : bb == 2 ? acc[a][2][r] : acc[a][3][r];
                }
                // keep the next rows' loads from being hoisted here (register pressure)
                if ((r & 3) == 3) asm volatile("" ::: "memory");
            }
        }
        asm volatile("" ::: "memory");
        double sum = 0.0;
        {
            const double2 *dp = reinterpret_cast<const double2 *>(area + lane * kEpiRowB);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const double2 v = dp[q];
                sum += v.x;
                sum += v.y;
            }
        }
        if (row_j < M) {
            const long long at = static_cast<long long>(row_j) * o.segs + seg;
            o.part_R[at] = mrow == ninf ? ninf : Rj;
            o.part_s[at] = sum;
        }
    }
#undef SV_RL
}

template <int EPI>
hipError_t lm_launch(const void *H, const void *W, int M, int D, int V, const LmOut &o, hipStream_t s) {
    const int mtiles = (M + kTM - 1) / kTM;
    const int ntiles = (V + kTN - 1) / kTN;
    const long long blocks = static_cast<long long>(kXcds) * mtiles * ((ntiles + kXcds - 1) / kXcds);
    return launch_kernel(k_lmhead<EPI>, dim3(static_cast<unsigned>(blocks)), dim3(kLmThreads), 0, s,
                         static_cast<const uint4 *>(H), static_cast<const uint4 *>(W), M, D, V, mtiles,
                         ntiles, o);
}

}  // namespace

int lmhead_segs(int V) { return (V + kSegCols - 1) / kSegCols; }

hipError_t launch_lmhead_argmax(const void *H, const void *W, int M, int D, int V, uint64_t *part_k,
                                hipStream_t s) {
    LmOut o{};
    o.segs = lmhead_segs(V);
    o.keys = part_k;
    return lm_launch<kEpiArgmax>(H, W, M, D, V, o, s);
}

hipError_t launch_lmhead_stats(const void *H, const void *W, int B, int K, int D, int V,
                               const int32_t *drafts, const Scale &sc, float *part_R, double *part_s,
                               float *xlog, hipStream_t s) {
    LmOut o{};
    o.segs = lmhead_segs(V);
    o.part_R = part_R;
    o.part_s = part_s;
    o.xlog = xlog;
    o.drafts = drafts;
    o.K = K;
    o.c_hi = sc.c_hi;
    o.c_lo = sc.c_lo;
    return lm_launch<kEpiStats>(H, W, B * (K + 1), D, V, o, s);
}

hipError_t launch_lmhead_rows(const void *H, const void *W, int B, int K, int D, int V,
                              const ResidParam *rp, float *rows, hipStream_t s) {
    LmOut o{};
    o.segs = lmhead_segs(V);
    o.K = K;
    o.rp = rp;
    o.rows = rows;
    return lm_launch<kEpiRows>(H, W, B, D, V, o, s);
}

}  // namespace sv
