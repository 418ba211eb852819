// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qwg_internal.h"

namespace qwg {

// fp16 bit patterns held in the low / high half of a 32-bit register, widened to
// fp32. Used as FMA operands, the compiler folds the widening into
// v_fma_mix_f32 (one VALU op per weight).
__device__ __forceinline__ float h2f_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float h2f_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// True if v converts to fp16 and back unchanged (the GEMV engines keep their
// codebook tables in fp16; a value that fp16 cannot hold would be rounded).
__device__ __forceinline__ bool fp16_exact(float v) { return (float)(_Float16)v == v; }

// Wave-uniform read-only activations are read through the constant address
// space, so the compiler fetches them with scalar loads into SGPRs (one operand
// of every VALU FMA) instead of per-lane vector loads.
typedef const __attribute__((address_space(4))) float *cfloat_p;
__device__ __forceinline__ cfloat_p as_scalar(const float *p) { return (cfloat_p)p; }

// Problem descriptors and workgroup maps of a grouped launch are read through
// the constant address space (scalar loads).
typedef const __attribute__((address_space(4))) GemvArgs *cargs_p;
typedef const __attribute__((address_space(4))) uint32_t *cu32_p;

__device__ __forceinline__ void load_args(GemvArgs &a, cargs_p pa) {
    a.w = pa->w;
    a.x = pa->x;
    a.grid = pa->grid;
    a.y = pa->y;
    a.partial = pa->partial;
    a.counters = pa->counters;
    a.row_bytes = pa->row_bytes;
    a.n_in = pa->n_in;
    a.n_out = pa->n_out;
    a.nb = pa->nb;
    a.tiles = pa->tiles;
    a.splits = pa->splits;
    a.wg_begin = pa->wg_begin;
    a.layout = pa->layout;
}

// Asynchronous 16-byte global -> LDS copy (LDS DMA) of every active lane: lane
// i's 16 bytes land at LDS byte address lds + 16*i. Issued from inline asm so
// that the compiler does not guard later LDS reads with a wait for all
// outstanding loads; the kernels count these copies themselves (wait_vmcnt).
// The leading s_nop covers the M0-write -> LDS-DMA hazard.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"{m0}"(lds), "v"(g) : "memory");
}

// Streaming variant for whole lines read once (tile-layout weights): the
// non-temporal hint keeps them from displacing reused data in the caches.
// Measured on MI355X with a pure LDS-DMA stream (8 KB stages, 1536-2048
// workgroups): 6.0-6.4 TB/s without the hint, 6.7-7.1 TB/s with it; the
// grouped C5 Q4_K tile stream 101.6 -> 88.4 us, the IQ3 one 118 -> 96 us.
#ifndef QWG_STREAM_HINT
#define QWG_STREAM_HINT "nt"
#endif
__device__ __forceinline__ void dma16_stream(const void *g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off " QWG_STREAM_HINT ::"{m0}"(lds),
                 "v"(g)
                 : "memory");
}

// The same with a 64-bit scalar base and a 32-bit per-lane byte offset.
// The base must be wavefront-uniform; readfirstlane states that to the compiler
// (it folds away where uniformity is already known).
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    // (readfirstlane returns int: widen through uint32_t, never by sign extension)
    const uint64_t p = (uint64_t)(uintptr_t)sbase;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint64_t u = (uint64_t)lo | (uint64_t)hi << 32;
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"{m0}"(lds), "v"(voff),
                 "s"((const void *)(uintptr_t)u)
                 : "memory");
}

// Loads from an absolute LDS byte address (kernels whose dynamic LDS is their
// only LDS, so it starts at address 0). The address goes straight into the
// ds_read instruction, with no base register to add.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ T lds_load(uint32_t addr) {
    return *(const __attribute__((address_space(3))) T *)(size_t)addr;
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait_vmcnt with a wavefront-uniform count in 0..7 (larger counts wait for
// everything, which is always safe).
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
    switch (__builtin_amdgcn_readfirstlane(n)) {
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

// Workgroup barrier after this wavefront's LDS and scalar operations have
// completed; outstanding vector-memory operations (LDS DMA) are not waited for.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Constants hidden from the optimizer so that mask-and-convert patterns are
// kept as written (otherwise the compiler rewrites byte masks into per-field
// bit extracts, one more op per weight).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// First position from k on (k, k + stride, ...) that holds work, or a
// position >= nitems.
__device__ __forceinline__ int skip_holes(int k, int stride, int nitems, const GroupArgs &g) {
    if (g.tile != nullptr)
        while (k < nitems && ((cu32_p)g.map)[k] == kNoItem) k += stride;
    return k;
}

// End of a 64-row tile for one workgroup: `total` is this lane's row sum over
// the workgroup's super-block range (batch element `bt`). With one split the
// row is stored directly. Otherwise every split stores its partial, and the
// workgroup that arrives last at the tile's counter sums the partials in split
// order (so the result does not depend on arrival order), stores the rows and
// re-arms the counter for the next launch. Executed by one full wavefront.
//
// Cross-workgroup visibility without cache maintenance: the partials are
// written and read with agent-scope atomic stores/loads (coherent across the
// XCDs' L2 caches), and the wavefront waits for its stores to complete before it
// increments the counter; the last workgroup reads them only after its counter
// update has returned. An agent-scope fence would instead write back and
// invalidate the whole L2 of the XCD for every workgroup.
// Eight agent-coherent 4-byte loads (the form a relaxed agent-scope atomic
// load takes on this target), issued back to back with one wait for all.
__device__ __forceinline__ void load8_agent(const float *const (&p)[8], float (&v)[8]) {
    asm volatile(
        "global_load_dword %0, %8, off sc1\n\t"
        "global_load_dword %1, %9, off sc1\n\t"
        "global_load_dword %2, %10, off sc1\n\t"
        "global_load_dword %3, %11, off sc1\n\t"
        "global_load_dword %4, %12, off sc1\n\t"
        "global_load_dword %5, %13, off sc1\n\t"
        "global_load_dword %6, %14, off sc1\n\t"
        "global_load_dword %7, %15, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
        : "memory");
}

template <int NB>
__device__ __forceinline__ void tile_epilogue(const GemvArgs &a, int tile, int split,
                                              const float (&total)[NB]) {
    const int lane = threadIdx.x & 63;
    const int row = tile * kTileRows + lane;
    if (a.splits == 1) {
        if (row < a.n_out) {
#pragma unroll
            for (int bt = 0; bt < NB; ++bt) a.y[(int64_t)bt * a.n_out + row] = total[bt];
        }
        return;
    }
    const int64_t plane = (int64_t)a.tiles * kTileRows;
#pragma unroll
    for (int bt = 0; bt < NB; ++bt)
        __hip_atomic_store(&a.partial[((int64_t)split * NB + bt) * plane + row], total[bt],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The partials must have reached the coherence point before the count is
    // taken: wait for every outstanding memory operation of this wavefront.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    uint32_t old = 0;
    if (lane == 0)
        old = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (uint32_t)(a.splits - 1)) return;
    // Sum in split order. The partials are fetched eight at a time by one asm
    // block (agent-coherent loads, one wait): eight splits of one vector, or
    // the NB vectors of one split. The compiler keeps atomic loads in order
    // and waited one memory round trip per load (measured: 15 us for 22
    // splits of one launch).
    float acc[NB];
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) acc[bt] = 0.0f;
    if constexpr (NB == 1) {
        for (int s0 = 0; s0 < a.splits; s0 += 8) {
            const float *p[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                p[u] = &a.partial[(int64_t)(s0 + u < a.splits ? s0 + u : s0) * plane + row];
            float v[8];
            load8_agent(p, v);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < a.splits) acc[0] += v[u];
        }
    } else {
        // one batch of loads per split: its NB values (padded to eight)
        for (int s = 0; s < a.splits; ++s) {
            const float *p[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                p[u] = &a.partial[((int64_t)s * NB + (u < NB ? u : NB - 1)) * plane + row];
            float v[8];
            load8_agent(p, v);
#pragma unroll
            for (int bt = 0; bt < NB; ++bt) acc[bt] += v[bt];
        }
    }
    if (row < a.n_out) {
#pragma unroll
        for (int bt = 0; bt < NB; ++bt) a.y[(int64_t)bt * a.n_out + row] = acc[bt];
    }
    if (lane == 0)
        __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qwg
