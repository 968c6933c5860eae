// sv_device.hpp -- device-side building blocks shared by the verification kernels:
// 16-byte logit loaders, bf16 widening, and wave64 reductions / scans.
//
// All reductions here are fixed-order (butterfly or Hillis-Steele over lane
// ids), so every kernel built on them is deterministic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

// Element type tags: logits are either IEEE binary32 or bfloat16 bit patterns.
struct F32 {
    using storage = float;
    static constexpr int kPerVec = 4;                   // elements per 16-byte vector
    static constexpr uint32_t kNegInfWord = 0xff800000u;  // one -inf per dword
};
struct BF16 {
    using storage = uint16_t;
    static constexpr int kPerVec = 8;
    static constexpr uint32_t kNegInfWord = 0xff80ff80u;  // two bf16 -inf per dword
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t h) { return bf16_to_f32(h); }
// A stored element's bits, and the element from them.
__device__ __forceinline__ unsigned storage_bits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ unsigned storage_bits(uint16_t h) { return h; }
template <typename E>
__device__ __forceinline__ float from_bits(unsigned u) {
    if constexpr (sizeof(typename E::storage) == 2)
        return bf16_to_f32(static_cast<uint16_t>(u));
    else
        return __uint_as_float(u);
}

// Unpack one 16-byte vector into kPerVec floats (exact widening).
__device__ __forceinline__ void unpack(const uint4 &w, float (&x)[4]) {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
}
__device__ __forceinline__ void unpack(const uint4 &w, float (&x)[8]) {
    // bf16 pairs: the low half is the earlier element.
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
    x[4] = __uint_as_float(w.z << 16);
    x[5] = __uint_as_float(w.z & 0xffff0000u);
    x[6] = __uint_as_float(w.w << 16);
    x[7] = __uint_as_float(w.w & 0xffff0000u);
}

// Vector j (kPerVec consecutive elements) of a row of V logits.  ALIGNED means
// the row starts on a 16-byte boundary and V is a multiple of kPerVec, so the
// vector is one 16-byte load.  Otherwise elements are loaded one by one and
// those at or past V read as -inf.
template <typename E, bool ALIGNED>
__device__ __forceinline__ void load_vec(const typename E::storage *__restrict__ row, int V, int j,
                                         float (&x)[E::kPerVec]) {
    if constexpr (ALIGNED) {
        const uint4 w = reinterpret_cast<const uint4 *>(row)[j];
        unpack(w, x);
    } else {
#pragma unroll
        for (int e = 0; e < E::kPerVec; ++e) {
            const int idx = j * E::kPerVec + e;
            x[e] = idx < V ? to_f32(row[idx]) : -__builtin_huge_valf();
        }
    }
}

// A 16-byte vector held in registers between its load and its use, so a wave
// can issue all of its loads before consuming any of them.  The aligned form
// keeps the raw 16 bytes (4 VGPRs); the general form keeps widened floats.
template <typename E, bool ALIGNED>
struct Staged;

// Streamed logits are read once: non-temporal loads keep them from displacing
// useful lines (measured: +8% read bandwidth on MI355X for these passes).
#ifndef SV_NT_LOADS
#define SV_NT_LOADS 1
#endif
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename E>
struct Staged<E, true> {
    uint4 w;
    __device__ __forceinline__ void load(const typename E::storage *__restrict__ row, int, int j) {
#if SV_NT_LOADS
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row) + j);
        w = make_uint4(v.x, v.y, v.z, v.w);
#else
        w = reinterpret_cast<const uint4 *>(row)[j];
#endif
    }
    __device__ __forceinline__ void set_neg_inf() {
        w = make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
    }
    __device__ __forceinline__ void get(float (&x)[E::kPerVec]) const { unpack(w, x); }
};

template <typename E>
struct Staged<E, false> {
    float v[E::kPerVec];
    __device__ __forceinline__ void load(const typename E::storage *__restrict__ row, int V, int j) {
        load_vec<E, false>(row, V, j, v);
    }
    __device__ __forceinline__ void set_neg_inf() {
#pragma unroll
        for (int e = 0; e < E::kPerVec; ++e) v[e] = -__builtin_huge_valf();
    }
    __device__ __forceinline__ void get(float (&x)[E::kPerVec]) const {
#pragma unroll
        for (int e = 0; e < E::kPerVec; ++e) x[e] = v[e];
    }
};

// Four consecutive elements of a row (vector j holds elements 4j..4j+3),
// widened to fp32: a row of type E read in step with an fp32 row.  For fp32 it
// is Staged; for bf16 the aligned form is one 8-byte load (row 8-byte aligned,
// V % 4 == 0).
template <typename E, bool ALIGNED>
struct Staged4 : Staged<E, ALIGNED> {
    static_assert(E::kPerVec == 4, "fp32 rows are Staged as they are");
};

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <>
struct Staged4<BF16, true> {
    uint2 w;
    __device__ __forceinline__ void load(const uint16_t *__restrict__ row, int, int j) {
#if SV_NT_LOADS
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(row) + j);
        w = make_uint2(v.x, v.y);
#else
        w = reinterpret_cast<const uint2 *>(row)[j];
#endif
    }
    __device__ __forceinline__ void set_neg_inf() { w = make_uint2(BF16::kNegInfWord, BF16::kNegInfWord); }
    __device__ __forceinline__ void get(float (&x)[4]) const {
        x[0] = __uint_as_float(w.x << 16);
        x[1] = __uint_as_float(w.x & 0xffff0000u);
        x[2] = __uint_as_float(w.y << 16);
        x[3] = __uint_as_float(w.y & 0xffff0000u);
    }
};

template <>
struct Staged4<BF16, false> {
    float v[4];
    __device__ __forceinline__ void load(const uint16_t *__restrict__ row, int V, int j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = j * 4 + e;
            v[e] = idx < V ? bf16_to_f32(row[idx]) : -__builtin_huge_valf();
        }
    }
    __device__ __forceinline__ void set_neg_inf() {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = -__builtin_huge_valf();
    }
    __device__ __forceinline__ void get(float (&x)[4]) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = v[e];
    }
};

// Fixed-order pairwise sum of a small array.
template <int P>
__device__ __forceinline__ float pairwise_sum(float (&a)[P]) {
#pragma unroll
    for (int w = P / 2; w >= 1; w /= 2) {
#pragma unroll
        for (int i = 0; i < w; ++i) a[i] = a[i] + a[i + w];
    }
    return a[0];
}

// ---- wave64 reductions ------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// One DPP step of a row (16-lane) reduction on a double: v + v[lane ^ ...]
// for the given row-local pattern, moved as two 32-bit halves.
template <int CTRL>
__device__ __forceinline__ double row_step(double v) {
    const unsigned long long u = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, 0xf, 0xf, false);
    return v + __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) |
                                                          static_cast<unsigned>(lo)));
}

// The totals of two per-lane values over the wave, with cross-lane moves only
// (no LDS round trips): lanes 0..31 end with a's total, lanes 32..63 with b's.
// The half-wave swap puts a's two halves beside each other in lanes 0..31 and
// b's in 32..63 (one add then leaves 32 partials of each), the row swap pairs
// rows 0 with 1 and 2 with 3, and four DPP steps (neighbour, pair of
// neighbours, half-row mirror, row mirror) finish each row.
__device__ __forceinline__ double wave_sum_pair(double a, double b) {
    const unsigned long long ua = __double_as_longlong(a), ub = __double_as_longlong(b);
    const auto lo = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(ua), static_cast<unsigned>(ub), false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(ua >> 32), static_cast<unsigned>(ub >> 32),
                                                     false, false);
    auto join = [](unsigned l, unsigned h) {
        return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(h) << 32) | l));
    };
    double v = join(lo[0], hi[0]) + join(lo[1], hi[1]);
    const unsigned long long uv = __double_as_longlong(v);
    const auto lo2 = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(uv), static_cast<unsigned>(uv), false, false);
    const auto hi2 = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(uv >> 32), static_cast<unsigned>(uv >> 32),
                                                      false, false);
    v = join(lo2[0], hi2[0]) + join(lo2[1], hi2[1]);
    v = row_step<0xb1>(v);   // quad_perm [1, 0, 3, 2]
    v = row_step<0x4e>(v);   // quad_perm [2, 3, 0, 1]
    v = row_step<0x141>(v);  // row_half_mirror
    v = row_step<0x140>(v);  // row_mirror
    return v;
}

// Inclusive prefix sum over lanes (Hillis-Steele; fixed order).
__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double y = __shfl_up(v, o, kWave);
        if (lane >= o) v += y;
    }
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t y = __shfl_xor(v, o, kWave);
        v = y > v ? y : v;
    }
    return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }


// (value, index) packed so that the larger key has the larger value and, among
// equal values, the lower index.  -0 is folded into +0 so that the two compare
// equal, as floats do; NaN is not ordered meaningfully (inputs are finite or -inf).
__device__ __forceinline__ uint64_t argmax_key(float v, int idx) {
    uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return (static_cast<uint64_t>(b) << 32) | static_cast<uint32_t>(0xffffffffu - static_cast<uint32_t>(idx));
}
__device__ __forceinline__ int argmax_key_index(uint64_t k) {
    return static_cast<int>(0xffffffffu - static_cast<uint32_t>(k & 0xffffffffu));
}

// Lowest / highest set lane of a non-zero mask.
__device__ __forceinline__ int first_lane(uint64_t m) { return __ffsll(static_cast<long long>(m)) - 1; }
__device__ __forceinline__ int last_lane(uint64_t m) { return 63 - __clzll(static_cast<long long>(m)); }

// exp2 on the hardware transcendental unit (v_exp_f32); -inf gives 0.
__device__ __forceinline__ float fast_exp2(float a) { return __builtin_amdgcn_exp2f(a); }

// ---- cross-wave hand-off inside one kernel ----------------------------------------
//
// Waves of one launch that pass words to each other (segment partials, row
// normalisers, a request's decision state) use device-scope atomic loads and
// stores for those words: the hardware keeps them coherent across the XCDs'
// separate L2 caches without the whole-cache write-back and invalidation a
// device-scope fence costs there (tens of microseconds per fence, measured).
// The one ordering needed - a wave's shared stores complete before the atomic
// that publishes its decision - comes from waiting on the wave's own
// outstanding memory operations.  A wave waits for another only by polling a
// word written once, by a wave dispatched before it, which either writes it
// or, having found the request settled, lets the poller find that too.
//
// Why that is enough on gfx950.  In the LLVM AMDGPU memory model for
// GFX942/GFX950, an agent-scope release is "buffer_wbl2 sc1; s_waitcnt
// vmcnt(0)" before the releasing operation, and an agent-scope acquire is
// "s_waitcnt vmcnt(0); buffer_inv sc1" after the acquiring one.  The L2
// write-back and invalidate are there for ordinary (non-atomic) stores and
// loads, which may sit in one XCD's L2.  Every word this hand-off shares is
// written and read with agent-scope atomic instructions instead: relaxed
// agent-scope loads and stores are emitted with the sc1 bit (the memory
// model's coherent form for that scope) and read-modify-writes as global
// atomics, the same instructions an acquire or release would use.  So the
// release needs only the wait: on this gfx9-family part vmcnt counts stores
// and atomics as well as loads, and it drops only when the memory system has
// acknowledged them.  On the reading side, the loads of another wave's words
// are control-dependent on the value a poll returned or on the returned value
// of the mask atomic (the branch that selects the deciding or finishing wave
// needs it), and a wave issues in order without speculating past a branch, so
// they issue after it returns; the logits they then read are inputs no kernel
// of the launch writes.
// The waiting is an asm statement with a memory clobber, so the compiler can
// move no memory access across it either.

template <typename T>
__device__ __forceinline__ void shared_store(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T shared_load(T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_own_stores() {
    asm volatile("s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0)" ::: "memory");
}

// Values every lane holds alike, moved to a scalar register so branches on
// them are uniform.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ unsigned uniform(unsigned v) {
    return static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}
__device__ __forceinline__ uint64_t uniform(uint64_t v) {
    const unsigned lo = uniform(static_cast<unsigned>(v)), hi = uniform(static_cast<unsigned>(v >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

}  // namespace sv
