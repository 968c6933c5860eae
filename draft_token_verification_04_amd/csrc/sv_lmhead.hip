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
// bf16, both k-contiguous.  A workgroup of 4 waves owns a 256 x 256 tile of C
// and walks D in steps of 64: the next step's H and W slabs are loaded into
// registers while the current one is multiplied out of LDS (two LDS buffers,
// rows padded to 144 bytes so the fragment reads hit distinct banks), then
// stored to the other buffer; one barrier per step.  Each wave holds a
// 128 x 128 quarter as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16 accumulators
// (fp32).  Workgroups are numbered so that the 8 row tiles of one column tile
// run together on one XCD (consecutive workgroup ids go to consecutive XCDs):
// the column tile's W slab is then read from HBM once and shared through that
// XCD's L2.
#include <limits.h>

#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;
constexpr int kTM = 256, kTN = 256, kTK = 64;  // workgroup tile and D step
constexpr int kRowBytes = kTK * 2 + 16;        // LDS bytes per tile row (padded)
constexpr int kTileBytes = kTM * kRowBytes;    // one operand slab in LDS
constexpr int kSegCols = 128;                  // columns per argmax key (one wave's width)
constexpr int kLoadsPerThread = kTM * kTK * 2 / 16 / kBlock;  // 16-byte chunks per operand

__device__ __forceinline__ bf16x8 lds_frag(const char *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

__global__ __launch_bounds__(kBlock, 1) void k_lmhead_argmax(const uint4 *__restrict__ H,
                                                             const uint4 *__restrict__ W, int M, int D,
                                                             int V, int mtiles, int ntiles,
                                                             uint64_t *__restrict__ part_k, int segs) {
    __shared__ __align__(16) char lds[4 * kTileBytes];  // [stage][A|B]
    const int bid = blockIdx.x;
    const int xcd = bid % kXcds, j = bid / kXcds;
    const int mt = j % mtiles;
    const int nt = (j / mtiles) * kXcds + xcd;
    if (nt >= ntiles) return;
    const int m0 = mt * kTM, n0 = nt * kTN;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int dv = D / 8;  // 16-byte chunks per row

    // global -> register staging: chunk q = tid + kBlock*i is row q/8, column
    // chunk q%8; offsets are 32-bit element counts from the uniform bases
    // (H and W rows past M or V read the last row instead)
    const int r0 = tid >> 3, c0 = tid & 7;
    int ga[kLoadsPerThread], gb[kLoadsPerThread];
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
        ga[i] = min(m0 + r0 + 32 * i, M - 1) * dv + c0;
        gb[i] = min(n0 + r0 + 32 * i, V - 1) * dv + c0;
    }
    char *const st0 = lds + r0 * kRowBytes + c0 * 16;  // this thread's slot in stage 0's A slab

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    // fragment offsets: lane reads 8 k-values of row (l % 32) at k offset 8 (l / 32)
    const int fa = (wm * 128 + (lane & 31)) * kRowBytes + (lane >> 5) * 16;
    const int fb = (wn * 128 + (lane & 31)) * kRowBytes + (lane >> 5) * 16;
    const int nk = D / kTK;
    uint4 ra[kLoadsPerThread], rb[kLoadsPerThread];
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
        ra[i] = H[ga[i]];
        rb[i] = W[gb[i]];
    }
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
        *reinterpret_cast<uint4 *>(st0 + i * 32 * kRowBytes) = ra[i];
        *reinterpret_cast<uint4 *>(st0 + kTileBytes + i * 32 * kRowBytes) = rb[i];
    }
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        // the next step's slabs (the last step loads its own again; never read)
        const int kn = min(s + 1, nk - 1) * (kTK / 8);
#pragma unroll
        for (int i = 0; i < kLoadsPerThread; ++i) {
            ra[i] = H[ga[i] + kn];
            rb[i] = W[gb[i] + kn];
        }
        const char *sa = lds + (s & 1) * 2 * kTileBytes, *sb = sa + kTileBytes;
#pragma unroll
        for (int kk = 0; kk < kTK / 16; ++kk) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                af[t] = lds_frag(sa + fa + t * 32 * kRowBytes + kk * 32);
                bfr[t] = lds_frag(sb + fb + t * 32 * kRowBytes + kk * 32);
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
        }
        char *dn = st0 + ((s + 1) & 1) * 2 * kTileBytes;
#pragma unroll
        for (int i = 0; i < kLoadsPerThread; ++i) {
            *reinterpret_cast<uint4 *>(dn + i * 32 * kRowBytes) = ra[i];
            *reinterpret_cast<uint4 *>(dn + kTileBytes + i * 32 * kRowBytes) = rb[i];
        }
        __syncthreads();
    }

    // epilogue: per row, the first maximum over this wave's 128 columns
    const int seg = (n0 + wn * 128) / kSegCols;
    if (seg >= segs) return;
    const int cbase = n0 + wn * 128 + (lane & 31);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
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
            const int row = m0 + wm * 128 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
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
    return launch_kernel(k_lmhead_argmax, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s,
                         static_cast<const uint4 *>(H), static_cast<const uint4 *>(W), M, D, V, mtiles,
                         ntiles, part_k, lmhead_segs(V));
}

}  // namespace sv
