// sv_probe.hip -- a read-only streaming kernel that gives the HBM read rate
// this device actually reaches, the practical ceiling the verification passes
// are compared against (the published 8 TB/s is a pin rate, not a read rate).
//
// Each wave reads kProbeVecs 16-byte vectors per lane (16 KB) with the same
// non-temporal, fully coalesced loads as the row passes (64 consecutive
// vectors per load instruction), issues them all before using any, and writes
// the XOR of its 4096 words: one word per 16 KB read, so every load is used
// and the writes are 1/4096 of the traffic.  Workgroups of 8 waves: in a sweep
// of 4..32 vectors per lane, 256..1024 threads and persistent grids this shape
// was within 1% of the best read rate (about 7.0 TB/s on MI355X).
#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {
namespace {

constexpr int kProbeVecs = 16;  // vectors per lane (16 KB per wave)
constexpr int kProbeBlock = 512;
constexpr int kProbeWavesPerBlock = kProbeBlock / kWave;

__global__ __launch_bounds__(kProbeBlock) void k_read_probe(const u32x4 *__restrict__ p, long long n16,
                                                       long long nwaves, unsigned *__restrict__ folds) {
    const int lane = threadIdx.x & (kWave - 1);
    const long long wave = static_cast<long long>(blockIdx.x) * kProbeWavesPerBlock + (threadIdx.x >> 6);
    if (wave >= nwaves) return;
    const long long base = wave * (kWave * kProbeVecs) + lane;
    u32x4 v[kProbeVecs];
#pragma unroll
    for (int j = 0; j < kProbeVecs; ++j) {
        const long long i = base + static_cast<long long>(j) * kWave;
        v[j] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
    }
    unsigned f = 0;
#pragma unroll
    for (int j = 0; j < kProbeVecs; ++j) f ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) f ^= static_cast<unsigned>(__shfl_xor(static_cast<int>(f), o, kWave));
    if (lane == 0) folds[wave] = f;
}

}  // namespace

long long read_probe_waves(long long n16) { return (n16 + kWave * kProbeVecs - 1) / (kWave * kProbeVecs); }

hipError_t launch_read_probe(const void *buf, long long n16, unsigned *folds, hipStream_t s) {
    const long long nwaves = read_probe_waves(n16);
    const long long blocks = (nwaves + kProbeWavesPerBlock - 1) / kProbeWavesPerBlock;
    return launch_kernel(k_read_probe, dim3(static_cast<unsigned>(blocks)), dim3(kProbeBlock), 0, s,
                         static_cast<const u32x4 *>(buf), n16, nwaves, folds);
}

}  // namespace sv
