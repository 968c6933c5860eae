// sv_lmhead.hip -- the target's LM-head projection fused with the row argmax
// of greedy verification: logits = H W^T are formed tile by tile on the matrix
// cores and reduced at once to (max, lowest index) keys per 128-column segment;
// the logits are never written.
//
// What it feeds: the speculative-decoding tutorial page, section
// "一轮推测解码究竟发生什么" (the target scores all gamma+1 positions in one
// parallel pass; greedy verification keeps drafts while they equal the target's
// argmax), and the DLite notes, section 2 (the D x V vocabulary projection is
// the cost a drafter avoids repeating per position).
//
// k_lmhead_argmax: C[m][n] = sum_k H[m][k] W[n][k] with H [M][D] and W [V][D]
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

__global__ __launch_bounds__(kLmThreads, 1) void k_lmhead_argmax(const uint4 *__restrict__ H,
                                                             const uint4 *__restrict__ W, int M, int D,
                                                             int V, int mtiles, int ntiles,
                                                             uint64_t *__restrict__ part_k, int segs) {
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
    // 32-bit 16-byte-chunk counts; rows past M or V read the last row.
    int ga0, ga1, ga2, ga3, gb0, gb1, gb2, gb3;
#define SV_GOFF(i, GA, GB)                                        \
    {                                                             \
        const int r = 8 * (kLmWaves * (i) + w) + lane / kChunks;  \
        const int c = (lane % kChunks) ^ ((r >> 1) & 7);          \
        GA = min(m0 + r, M - 1) * dv + c;                         \
        GB = min(n0 + r, V - 1) * dv + c;                         \
    }
    SV_GOFF(0, ga0, gb0)
    SV_GOFF(1, ga1, gb1)
    SV_GOFF(2, ga2, gb2)
    SV_GOFF(3, ga3, gb3)
#undef SV_GOFF
    static_assert(kDmaPerOperand == 4, "four DMA instructions per operand per wave");
    const int nk = D / kTK;
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

    // epilogue: per row, the first maximum over this wave's 128 columns
    const int seg = (n0 + wn * 128) / kSegCols;
    if (seg >= segs) return;
    const int cbase = n0 + wn * 128 + (lane & 31);
    const f32x16 acc[2][4] = {{c00, c01, c02, c03}, {c10, c11, c12, c13}};
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float best = -__builtin_huge_valf();
            int bi = INT_MAX;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int col = cbase + b * kTileRows;
                const float x = col < V ? acc[a][b][r] : -__builtin_huge_valf();
                if (x > best || (bi == INT_MAX && col < V)) {
                    best = x;
                    bi = col;
                }
            }
            uint64_t key = argmax_key(best, bi);
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) {
                const uint64_t y = __shfl_xor(key, o, kWave);
                key = y > key ? y : key;
            }
            const int row = m0 + wm * 64 + a * kTileRows + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if ((lane & 31) == 0 && row < M) part_k[static_cast<long long>(row) * segs + seg] = key;
        }
    }
}

}  // namespace

int lmhead_segs(int V) { return (V + kSegCols - 1) / kSegCols; }

hipError_t launch_lmhead_argmax(const void *H, const void *W, int M, int D, int V, uint64_t *part_k,
                                hipStream_t s) {
    const int mtiles = (M + kTM - 1) / kTM;
    const int ntiles = (V + kTN - 1) / kTN;
    const long long blocks = static_cast<long long>(kXcds) * mtiles * ((ntiles + kXcds - 1) / kXcds);
    return launch_kernel(k_lmhead_argmax, dim3(static_cast<unsigned>(blocks)), dim3(kLmThreads), 0, s,
                         static_cast<const uint4 *>(H), static_cast<const uint4 *>(W), M, D, V, mtiles,
                         ntiles, part_k, lmhead_segs(V));
}

}  // namespace sv
