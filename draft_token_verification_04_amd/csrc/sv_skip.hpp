// sv_skip.hpp -- control words and the decision protocol shared by the
// row-skipping passes of the stochastic and greedy chains.
//
// A chain's outputs never depend on the rows after its first rejected (or
// mismatched) draft: every draft after it is discarded, and the one drawn token
// comes from the rejected position's row.  A row-skipping pass is one launch
// over every (position p, request b, segment) in position-major order, so the
// segments of position p are handed out before those of p+1 (the requests of
// a position in an order that may be rotated, see skip_request).  A wave of a
// position after 0 first tests whether its request is settled (its finished
// flag, or a rejection already recorded at an earlier position, see
// skip_early) and skips its segment if so.  Every other wave of (b, p) leaves
// its segment's partial in a word that starts at 0 and is never 0 once
// written, and ends; the wave of the last segment, dispatched after them,
// polls for those words (a word that never comes belongs to a wave that found
// the request settled, which the poller then finds too), takes the decision of
// position p and records it in the request's mask with one atomic OR: bit p =
// "position p decided", bit 32+p = "draft p rejected" (position K's bit means
// its bonus row is ready).  The request is decided once the mask holds a
// rejection with every earlier position decided, or every position 0..K
// decided without one; the decider whose OR turned that prefix from undecided
// to decided (exactly one can: see skip_prefix) finishes the request and
// raises the flag.  Rows of positions after the first rejection are read only
// by waves that started before the decision was known.
#pragma once

#include "sv_device.hpp"
#include "sv_internal.hpp"

namespace sv {

// Largest K the row-skipping passes handle (decided and rejected bits share one
// 64-bit word per request).
constexpr int kSkipMaxK = 31;

struct SkipCtl {
    uint64_t *mask;      // [B] decided | rejected << 32
    unsigned *finished;  // [B] raised after the request's outputs are written
    unsigned *lim;       // [B] last position whose row can be needed, from row samples (greedy
                         // chain only, whose workspace holds B more words than skip_ctl_bytes)
};

// True once a draft before position p is known rejected: only the rows up to
// a chain's first rejection are ever needed, so the rows of position p are
// dead, whether or not the positions before that rejection are decided yet.
// Read from the request's mask, which a decision updates at once (the request
// is finished only later, after its outputs are written).  Uniform; p <= 31.
//
// Which test a wave uses (this one, or the request's finished flag) depends
// on the bytes of one position's rows across the batch, see skip_early.
__device__ __forceinline__ bool skip_row_dead(const SkipCtl &ctl, int b, int p) {
    const uint64_t m = uniform(shared_load(&ctl.mask[b]));
    return (static_cast<unsigned>(m >> 32) & ((1u << p) - 1u)) != 0;
}

// Whether the row-skipping passes test the rejection bits (skip_row_dead)
// rather than the finished flag.  Measured on MI355X (greedy chain, K = 7, V =
// 151936 bf16): when one position's rows across the batch fit in what the chip
// keeps in flight (about 80 MB), retiring dead waves at once only moves the
// dispatch front sooner onto rows whose decisions have not landed, and the
// pass gets slower (B = 256, 78 MB: 86 us against 75 us; B = 320: 101 against
// 93); above that the earlier test saves reads and time (B = 384, 117 MB: 108
// against 109 us; B = 448: 116 against 122; B = 512: 124 against 130; the
// stochastic pass at B = 256, two rows per position, 156 MB: 147 against 150).
#ifndef SV_EARLY_SKIP_BYTES
#define SV_EARLY_SKIP_BYTES 110e6
#endif
constexpr double kEarlySkipPositionBytes = SV_EARLY_SKIP_BYTES;
inline bool skip_early(int B, int rows_per_position, int V, size_t elem) {
    return static_cast<double>(B) * rows_per_position * V * static_cast<double>(elem) >= kEarlySkipPositionBytes;
}

// Carves the control words of a B x K chain out of `base` without clearing
// them (the caller clears them together with other words).
void skip_ctl_carve(void *base, int B, int K, SkipCtl *ctl);

// The skip passes find a wave's position, request and segment with 32-bit
// scalar arithmetic (a few instructions, against a long 64-bit vector
// division every wave - the many that find their row settled included -
// would otherwise run first): the grid and the segment count must fit.
inline bool skip_grid_fits(long long waves, int segs) {
    return waves + kWavesPerBlock <= 0x7fffffffLL && segs >= 1 && segs <= 46340;
}

// This wave's index in the grid, as a scalar.
__device__ __forceinline__ unsigned skip_wave_index() {
    return blockIdx.x * static_cast<unsigned>(kWavesPerBlock) + uniform(static_cast<unsigned>(threadIdx.x >> 6));
}

// Vectors [v0, v1) of segment sg when a row's nvec vectors are cut into segs:
// v0 = floor(sg nvec / segs), computed as sg q + floor(sg r / segs) with
// (q, r) = nvec divmod segs, so that no product leaves 32 bits (segs <= 46340).
__device__ __forceinline__ void skip_segment(int sg, int nvec, int segs, int &v0, int &v1) {
    const unsigned q = static_cast<unsigned>(nvec) / static_cast<unsigned>(segs);
    const unsigned r = static_cast<unsigned>(nvec) - q * static_cast<unsigned>(segs);
    const unsigned s0 = static_cast<unsigned>(sg), s1 = s0 + 1u;
    v0 = static_cast<int>(s0 * q + (s0 * r) / static_cast<unsigned>(segs));
    v1 = static_cast<int>(s1 * q + (s1 * r) / static_cast<unsigned>(segs));
}

// Each position hands out its requests' rows in an order rotated by `rot`
// requests from the position before's: request b's row of position p comes
// at slot (b + p rot) mod B.  A decision lands about one position's span of
// reads after its row is handed out, so in plain order the next position's
// row of the same request is mostly handed out just before the decision that
// could skip it; rotated, a part of the requests get that row later (and the
// rest sooner).  Measured on MI355X (greedy chain, K = 7, V = 151936 bf16, us
// per pass, plain / rotated by B/2): B = 256 66.8 / 64.4, B = 320 80.6 /
// 75.7 with the finished-flag test; B = 384 89.5 / 93.0, B = 512 108.8 /
// 120.6, and the stochastic pass at B = 256 88.9 / 92, with the rejection-bit
// test (skip_early), which retires dead waves as soon as the rejection is
// known and gains nothing from the later hand-out.  The tree pass, over its
// depth-ranked node slots, at B = 64 with N = 33 (four workgroups per compute
// unit): 68.9-69.2 plain, 67.5 rotated by B/16, 67.7-68.0 by B/8, 68.3 by B/4
// or B/2.
inline int skip_rotation(int B, bool early) { return early ? 0 : B / 2; }
inline int tree_rotation(int B) { return B / 8; }
// The greedy chain, rotated, is faster still with the rejection-bit test
// (us per pass, rotated by B/2, finished flag / rejection bits): B = 256 64.9
// / 63.2, B = 320 76.0 / 76.6; without rotation the bits win from B = 384 on
// (see skip_early), and rotation there costs (B = 512: 109.4 against 120.5).
// So it always tests the bits and rotates where a position's rows are below
// the early-test threshold.  The stochastic pass keeps the flag below it (the
// bits with rotation: B = 32 34.0 against 32.2).
inline int greedy_rotation(int B, bool rotate) { return rotate ? B / 2 : 0; }

__device__ __forceinline__ int skip_request(unsigned slot, int p, int B, int rot) {
    if (rot == 0) return static_cast<int>(slot);
    // slot = (b + p rot) mod B, so b = (slot + p (B - rot)) mod B; p B < 2^31
    const unsigned b = (slot + static_cast<unsigned>(p) * static_cast<unsigned>(B - rot)) % static_cast<unsigned>(B);
    return static_cast<int>(b);
}

// The decided prefix of a request mask: the accepted length n once every
// position up to the first rejection (or every position 0..K) is decided, else
// -1.  Monotone: a mask with more bits set has the same prefix once it has one,
// so among the decisions recorded with atomic ORs exactly one turns it from -1
// into n.
__device__ __forceinline__ int skip_prefix(uint64_t m, int K) {
    const unsigned decided = static_cast<unsigned>(m), rejected = static_cast<unsigned>(m >> 32);
    if (rejected) {
        const int rj = __ffs(static_cast<int>(rejected)) - 1;
        const unsigned below = rj == 0 ? 0u : (0xffffffffu >> (32 - rj));
        return (decided & below) == below ? rj : -1;
    }
    const unsigned all = K == 31 ? 0xffffffffu : ((1u << (K + 1)) - 1u);
    return (decided & all) == all ? K : -1;
}

// Raises request b's flag once this wave's output stores are complete.
__device__ __forceinline__ void skip_finished(const SkipCtl &ctl, int b, int lane) {
    wait_own_stores();
    if (lane == 0) shared_store(&ctl.finished[b], 1u);
}

}  // namespace sv
