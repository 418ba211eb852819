// Device side of the short-call kernels (short.hip, iq3.hip): the end of a
// split tile through tagged words. Not installed.
//
// The grid is at most one workgroup per compute unit, so all of a
// launch's workgroups are resident at once on an idle device. Splits 0..S-2
// store their row sums as tagged 8-byte words (fp32 bits | tag << 32, one
// single-copy-atomic agent-scope store, no wait); split S-1 loads its peers'
// words, all in one round trip, until every tag is this call's, and adds them
// in split order. The tag is the tile's epoch + 1, where the epoch (one word
// per tile, read by every workgroup when it starts) is advanced by split S-1
// after it has used the words: a later launch, a graph replay included,
// starts after this one has ended and reads the new epoch. The wait is
// bounded (1 s); on giving up the rows are stored as NaN. (A tile's splits
// share an XCD, but polling through that XCD's L2 before the agent-coherent
// loads measured slower on back-to-back calls: 6.9 against 4.9 us for
// 2048 x 2048.)
#pragma once

#include "qwg_device.h"
#include "short_call.h"

namespace qwg {

namespace short_detail {

// 100 MHz constant clock: give up after 1 s.
constexpr uint64_t kShortWaitTicks = 100000000;

__device__ __forceinline__ void st_tagged(uint64_t *p, float v, uint32_t tag) {
    __hip_atomic_store(p, (uint64_t)__builtin_bit_cast(uint32_t, v) | ((uint64_t)tag << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Eight agent-coherent 8-byte loads back to back, one wait for all of them.
__device__ __forceinline__ void load8_words(const uint64_t *const (&p)[8], uint64_t (&v)[8]) {
    asm volatile(
        "global_load_dwordx2 %0, %8, off sc1\n\t"
        "global_load_dwordx2 %1, %9, off sc1\n\t"
        "global_load_dwordx2 %2, %10, off sc1\n\t"
        "global_load_dwordx2 %3, %11, off sc1\n\t"
        "global_load_dwordx2 %4, %12, off sc1\n\t"
        "global_load_dwordx2 %5, %13, off sc1\n\t"
        "global_load_dwordx2 %6, %14, off sc1\n\t"
        "global_load_dwordx2 %7, %15, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
        : "memory");
}

// Wavefront 0 of the workgroup: the tile's row sums `total` (this lane's row)
// of split `split` -> y.
__device__ __forceinline__ void short_epilogue(const GemvArgs &a, const ShortState &st, int tile,
                                               int split, uint32_t epoch, float total) {
    const int lane = threadIdx.x & 63;
    const int row = tile * kTileRows + lane;
    if (a.splits == 1) {
        if (row < a.n_out) a.y[row] = total;
        return;
    }
    const uint32_t tag = epoch + 1u;
    uint64_t *tw = st.words + (int64_t)tile * kShortMaxSplits * kTileRows;
    if (split != a.splits - 1) {
        st_tagged(&tw[split * kTileRows + lane], total, tag);
        return;
    }
    const int npeer = a.splits - 1;   // 1..7
    const uint64_t *p[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) p[s] = &tw[(s < npeer ? s : 0) * kTileRows + lane];
    uint64_t v[8];
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        load8_words(p, v);
        bool ok = true;
#pragma unroll
        for (int s = 0; s < 8; ++s) ok = ok && (s >= npeer || (uint32_t)(v[s] >> 32) == tag);
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > kShortWaitTicks) {
            if (row < a.n_out) a.y[row] = __builtin_nanf("");
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    float sum = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
        if (s < npeer) sum += __builtin_bit_cast(float, (uint32_t)v[s]);
    sum += total;
    if (row < a.n_out) a.y[row] = sum;
    if (lane == 0)
        __hip_atomic_store(&st.epochs[tile], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace short_detail

using short_detail::short_epilogue;

// (tile, split) of this workgroup in a short-call grid (short_grid); false for
// an idle position.
__device__ __forceinline__ bool short_item(const GemvArgs &a, int &tile, int &split) {
    const int kq = blockIdx.x >> 3;
    const int grp = kq / a.splits;
    tile = 8 * grp + (blockIdx.x & 7);
    split = kq - grp * a.splits;
    return tile < a.tiles;
}

}  // namespace qwg
