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
// 256 x 256 tile of C and walks D in steps of 32.  The H and W slabs of a step
// go straight from global memory into LDS (global_load_lds, 16 bytes per lane,
// no registers), issued three steps ahead into a ring of four LDS slots.  LDS
// rows are 64 bytes with the four 16-byte chunks of row r stored in the order
// c ^ ((r >> 2) & 3), so the fragment reads of 16 consecutive rows hit
// distinct banks.  Each wave holds a 64 x 128 part as 2 x 4 tiles of
// v_mfma_f32_32x32x16_bf16 accumulators (fp32).
//
// Schedule of step s (two 16-deep halves, h0 and h1):
//   read the h1 fragments of s; wait for the h0 fragments; MFMAs of h0;
//   wait for this wave's loads of step s + 1; barrier;
//   loads of step s + 3 into the slot of step s - 1; read the h0 fragments of
//   s + 1; wait for the h1 fragments of s; MFMAs of h1.
// The fragment reads of one half are thus always in flight under the MFMAs
// of the other, across the barrier too.  They are issued as inline ds_read
// instructions with explicit lgkmcnt waits tied to the fragment registers:
// with LDS DMA in flight the compiler would otherwise wait for every LDS read
// before each group of MFMAs.  The barrier of step s also means every wave
// has finished its reads of step s - 1, so that slot can be reloaded.
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
constexpr int kTM = 256, kTN = 256, kTK = 32;  // workgroup tile and D step
constexpr int kRowB = kTK * 2;                 // LDS bytes per slab row
constexpr int kSlab = kTM * kRowB;             // bytes of one operand slab (16 KB)
constexpr int kSlot = 2 * kSlab;               // one ring slot: the H slab, then the W slab
constexpr int kStages = 4;                     // ring slots; loads run kStages - 1 steps ahead
constexpr int kSegCols = 128;                  // columns per argmax key (one wave's width)
constexpr int kLmWaves = 8;
constexpr int kLmThreads = kLmWaves * kWave;
constexpr int kTileRows = 32;                  // rows (and columns) of one MFMA tile
constexpr int kLoadsPerStep = 4;               // 1 KB DMA instructions per wave per step

__shared__ __align__(1024) char ring[kStages * kSlot];

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

    // DMA mapping: the two instructions per operand of wave w fill slab rows
    // 16 q .. 16 q + 15 for q = w and q = 8 + w; lane l writes 16 bytes at
    // 16 l, i.e. row 16 q + l / 4, stored chunk l % 4, which holds the row's
    // logical chunk (l % 4) ^ ((row >> 2) & 3) (the swizzle is an involution).
    // Offsets are 32-bit 16-byte-chunk counts; rows past M or V read the last row.
    int ga0, ga1, gb0, gb1;
    {
        const int r0 = 16 * w + lane / 4, r1 = 16 * (8 + w) + lane / 4;
        const int c0 = (lane % 4) ^ ((r0 >> 2) & 3), c1 = (lane % 4) ^ ((r1 >> 2) & 3);
        ga0 = min(m0 + r0, M - 1) * dv + c0;
        ga1 = min(m0 + r1, M - 1) * dv + c1;
        gb0 = min(n0 + r0, V - 1) * dv + c0;
        gb1 = min(n0 + r1, V - 1) * dv + c1;
    }
    const int nk = D / kTK;  // a multiple of kStages (D % 128 == 0)
#define SV_ISSUE(S, step)                                                                                \
    {                                                                                                    \
        const int k0 = (step) * (kTK / 8);                                                               \
        char *sl = ring + (S) * kSlot;                                                                   \
        __builtin_amdgcn_global_load_lds(H + ga0 + k0, (SV_LDS void *)(sl + w * 1024), 16, 0, 0);        \
        __builtin_amdgcn_global_load_lds(W + gb0 + k0, (SV_LDS void *)(sl + kSlab + w * 1024), 16, 0, 0); \
        __builtin_amdgcn_global_load_lds(H + ga1 + k0, (SV_LDS void *)(sl + (8 + w) * 1024), 16, 0, 0);  \
        __builtin_amdgcn_global_load_lds(W + gb1 + k0, (SV_LDS void *)(sl + kSlab + (8 + w) * 1024), 16,   \
                                         0, 0);                                                          \
    }

    // Fragment addresses.  Lane l reads the 8 k-values of row (l % 32) of a
    // tile at k offset 8 (l / 32) within the half: logical chunk 2 h + l / 32,
    // stored at chunk (2 h + l / 32) ^ ((l >> 2) & 3) (tile rows are multiples
    // of 32, so the swizzle depends on the lane only).  Tile t of a slab sits
    // 2048 t bytes further; slot S adds S * kSlot, taken as an immediate offset
    // from a base for slots 0-1 and one 64 KB higher for slots 2-3.
    const uint32_t lbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SV_LDS char *)ring));
    const int sw = (lane >> 2) & 3;
    const uint32_t rowpart = static_cast<uint32_t>((lane & 31) * kRowB);
    const uint32_t a_h0 = lbase + wm * 64 * kRowB + rowpart + (((0 + (lane >> 5)) ^ sw) << 4);
    const uint32_t a_h1 = lbase + wm * 64 * kRowB + rowpart + (((2 + (lane >> 5)) ^ sw) << 4);
    const uint32_t b_h0 = lbase + kSlab + wn * 128 * kRowB + rowpart + (((0 + (lane >> 5)) ^ sw) << 4);
    const uint32_t b_h1 = lbase + kSlab + wn * 128 * kRowB + rowpart + (((2 + (lane >> 5)) ^ sw) << 4);
    const uint32_t a_h0_hi = a_h0 + 2 * kSlot, a_h1_hi = a_h1 + 2 * kSlot;
    const uint32_t b_h0_hi = b_h0 + 2 * kSlot, b_h1_hi = b_h1 + 2 * kSlot;

    f32x16 c00{}, c01{}, c02{}, c03{}, c10{}, c11{}, c12{}, c13{};
    bf16x8 p0, p1, q0, q1, q2, q3;  // fragments of the half in flight (A tiles 0-1, B tiles 0-3)
    bf16x8 r0, r1, t0, t1, t2, t3;  // fragments of the other half
#define SV_READ(S, HALF, A0, A1, B0, B1, B2, B3)                                                  \
    {                                                                                            \
        const uint32_t ab = ((S) < 2) ? ((HALF) ? a_h1 : a_h0) : ((HALF) ? a_h1_hi : a_h0_hi);  \
        const uint32_t bb = ((S) < 2) ? ((HALF) ? b_h1 : b_h0) : ((HALF) ? b_h1_hi : b_h0_hi);  \
        constexpr int so = ((S) & 1) * kSlot;                                                    \
        A0 = lds_read(ab, IC<so + 0 * 2048>{});                                                 \
        A1 = lds_read(ab, IC<so + 1 * 2048>{});                                                 \
        B0 = lds_read(bb, IC<so + 0 * 2048>{});                                                 \
        B1 = lds_read(bb, IC<so + 1 * 2048>{});                                                 \
        B2 = lds_read(bb, IC<so + 2 * 2048>{});                                                 \
        B3 = lds_read(bb, IC<so + 3 * 2048>{});                                                 \
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
#define SV_BARRIER() asm volatile("s_barrier" ::: "memory")

    SV_ISSUE(0, 0)
    SV_ISSUE(1, 1)
    SV_ISSUE(2, 2)
    wait_vm<2 * kLoadsPerStep>();  // this wave's loads of step 0 are done
    SV_BARRIER();                  // and every wave's
    SV_READ(0, 0, p0, p1, q0, q1, q2, q3)
    // step s in slot S (past the end, the last step is loaded again into a
    // slot nobody reads, and the h0 reads of the step after it are discarded)
#define SV_STEP(S)                                                        \
    SV_READ(S, 1, r0, r1, t0, t1, t2, t3)                                 \
    LDS_WAIT6(p0, p1, q0, q1, q2, q3);                                    \
    SV_MFMA(p0, p1, q0, q1, q2, q3)                                       \
    wait_vm<kLoadsPerStep>();                                             \
    SV_BARRIER();                                                         \
    SV_ISSUE(((S) + 3) % kStages, min(s + (S) + 3, nk - 1))               \
    SV_READ(((S) + 1) % kStages, 0, p0, p1, q0, q1, q2, q3)               \
    LDS_WAIT6(r0, r1, t0, t1, t2, t3);                                    \
    SV_MFMA(r0, r1, t0, t1, t2, t3)
    // no branches inside the ring (a branch makes the compiler wait for every load)
    for (int s = 0; s < nk; s += kStages) {
        SV_STEP(0)
        SV_STEP(1)
        SV_STEP(2)
        SV_STEP(3)
    }
#undef SV_STEP
#undef SV_MFMA
#undef SV_READ
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
