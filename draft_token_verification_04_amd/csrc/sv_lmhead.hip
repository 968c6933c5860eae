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
// no registers), issued three steps ahead into a ring of four LDS buffers; a
// step waits only for its own loads (vmcnt), then one barrier.  LDS rows are
// 64 bytes with the four 16-byte chunks of row r stored in the order
// c ^ ((r >> 2) & 3), so the fragment reads of 16 consecutive rows hit
// distinct banks.  Each wave holds a 64 x 128 part as 2 x 4 tiles of
// v_mfma_f32_32x32x16_bf16 accumulators (fp32).  Workgroups are numbered so
// that the row tiles of one column tile run together on one XCD (consecutive
// workgroup ids go to consecutive XCDs): the column tile's W slab is then read
// from HBM once and shared through that XCD's L2.
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
constexpr int kChunks = kRowB / 16;            // 16-byte chunks per slab row (4)
constexpr int kRowsPerDma = 1024 / kRowB;      // slab rows one wave-wide DMA fills (16)
constexpr int kSlab = kTM * kRowB;             // bytes of one operand slab
constexpr int kSegCols = 128;                  // columns per argmax key (one wave's width)
constexpr int kStages = 4;  // LDS ring slots; loads run kStages - 1 steps ahead
// Waves per workgroup: 4 (one per SIMD, 128 x 128 each) or 8 (two per SIMD,
// 64 x 128 each, so one wave's waits can hide behind the other's MFMAs).
#ifndef SV_LMHEAD_WAVES
#define SV_LMHEAD_WAVES 8
#endif
constexpr int kLmWaves = SV_LMHEAD_WAVES;
constexpr int kLmThreads = kLmWaves * kWave;
constexpr int kWavesM = kLmWaves / 2;          // waves along M (2 along N)
constexpr int kTilesA = kTM / kWavesM / 32;    // 32-row MFMA tiles per wave along M
constexpr int kDmaPerOperand = kSlab / 1024 / kLmWaves;  // 1 KB DMA instructions per wave per operand
constexpr int kLoadsPerStep = 2 * kDmaPerOperand;        // DMA loads per thread per step

// One array per ring slot and operand, so the compiler can tell which slot a
// fragment read touches and waits only for that slot's loads.
__shared__ __align__(1024) char sA0[kSlab], sA1[kSlab], sA2[kSlab], sA3[kSlab];
__shared__ __align__(1024) char sB0[kSlab], sB1[kSlab], sB2[kSlab], sB3[kSlab];
// Stored position of logical 16-byte chunk c of slab row r: consecutive rows
// rotate their chunks so that 16 lanes reading one logical chunk of 16
// consecutive rows hit 16 distinct 4-bank groups (measured: no bank conflicts).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 2) & 3); }
template <int S> __device__ __forceinline__ char *slab_a() {
    return S == 0 ? sA0 : S == 1 ? sA1 : S == 2 ? sA2 : sA3;
}
template <int S> __device__ __forceinline__ char *slab_b() {
    return S == 0 ? sB0 : S == 1 ? sB1 : S == 2 ? sB2 : sB3;
}
template <int S> using Slot = std::integral_constant<int, S>;

// vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

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

    // DMA mapping: instruction i of wave w fills slab rows kRowsPerDma q ..,
    // q = kLmWaves i + w; lane l writes 16 bytes at 16 l, i.e. row
    // kRowsPerDma q + l / kChunks, stored chunk l % kChunks, which holds the
    // row's logical chunk swz(r, l % kChunks) (the swizzle is an involution).
    // Offsets are 32-bit 16-byte-chunk counts; rows past M or V read the last row.
    int ga[kDmaPerOperand], gb[kDmaPerOperand];
#pragma unroll
    for (int i = 0; i < kDmaPerOperand; ++i) {
        const int r = kRowsPerDma * (kLmWaves * i + w) + lane / kChunks;
        const int c = swz(r, lane % kChunks);
        ga[i] = min(m0 + r, M - 1) * dv + c;
        gb[i] = min(n0 + r, V - 1) * dv + c;
    }
    auto issue = [&](auto slot, int step) {
        constexpr int S = decltype(slot)::value;
        const int k0 = step * (kTK / 8);
#pragma unroll
        for (int i = 0; i < kDmaPerOperand; ++i) {
            const int q = kLmWaves * i + w;
            __builtin_amdgcn_global_load_lds(H + ga[i] + k0, (SV_LDS void *)(slab_a<S>() + q * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(W + gb[i] + k0, (SV_LDS void *)(slab_b<S>() + q * 1024), 16, 0, 0);
        }
    };

    f32x16 acc[kTilesA][4];
#pragma unroll
    for (int a = 0; a < kTilesA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    // fragment reads: lane reads the 8 k-values of row (l % 32) at k offset 8 (l / 32)
    auto compute = [&](auto slot) {
        constexpr int S = decltype(slot)::value;
#pragma unroll
        for (int kk = 0; kk < kTK / 16; ++kk) {
            bf16x8 af[kTilesA], bfr[4];
            const int c = kk * 2 + (lane >> 5);
#pragma unroll
            for (int t = 0; t < kTilesA; ++t) {
                const int ra = wm * (kTilesA * 32) + t * 32 + (lane & 31);
                af[t] = *reinterpret_cast<const bf16x8 *>(slab_a<S>() + ra * kRowB + (swz(ra, c) << 4));
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int rb = wn * 128 + t * 32 + (lane & 31);
                bfr[t] = *reinterpret_cast<const bf16x8 *>(slab_b<S>() + rb * kRowB + (swz(rb, c) << 4));
            }
#pragma unroll
            for (int a = 0; a < kTilesA; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
        }
    };

    const int nk = D / kTK;  // a multiple of kStages (D % 128 == 0)
    issue(Slot<0>{}, 0);
    issue(Slot<1>{}, 1);
    issue(Slot<2>{}, 2);
    // step s: its loads are done once at most the kStages - 2 later steps'
    // loads are outstanding; the barrier then also means every wave has
    // finished step s - 1, whose slot the loads of step s + kStages - 1 reuse
    // (past the end, the last step is loaded again into a slot nobody reads)
#define SV_STEP(S)                                                            \
    wait_vm<(kStages - 2) * kLoadsPerStep>();                                 \
    __builtin_amdgcn_s_barrier();                                             \
    issue(Slot<(S + kStages - 1) % kStages>{}, min(s + S + kStages - 1, nk - 1)); \
    compute(Slot<S>{});
    // no branches inside the ring (a branch makes the compiler wait for every load)
    for (int s = 0; s < nk; s += kStages) {
        SV_STEP(0)
        SV_STEP(1)
        SV_STEP(2)
        SV_STEP(3)
    }
#undef SV_STEP
    wait_vm<0>();  // no DMA may still target LDS when the workgroup ends

    // epilogue: per row, the first maximum over this wave's 128 columns
    const int seg = (n0 + wn * 128) / kSegCols;
    if (seg >= segs) return;
    const int cbase = n0 + wn * 128 + (lane & 31);
#pragma unroll
    for (int a = 0; a < kTilesA; ++a) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float best = -__builtin_huge_valf();
            int bi = INT_MAX;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int col = cbase + b * 32;
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
            const int row = m0 + wm * (kTilesA * 32) + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
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
