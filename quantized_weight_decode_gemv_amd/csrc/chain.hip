// Layer-chain launch for gfx950: a decoder's per-token Q4_K weight stream as
// one persistent kernel whose phases run in dependency order.
//
// The order is the one of the "用 Python 重写 picoLM" page's model_forward /
// forward listings: per layer, q, k and v read the normalized x; the output
// projection reads the attention output; gate and up read the normalized
// residual; down reads silu(gate)*up; the next layer reads the updated x; the
// LM head reads the final norm. The norms, attention and activations between
// the products are not computed here, so a phase that depends on another waits
// for all of its outputs: the products of phase p+1 read their activations only
// after every workgroup has stored its results of phase p.
//
// One workgroup per compute unit, 16 wavefronts = 4 quads. A unit of work is
// one 64-row tile of one matrix over 1 or 2 super-block columns (tile layout:
// a column is 9216 contiguous bytes); each quad takes at most one unit per
// phase and computes it as the GEMV engines do (lane = row, wavefront G of the
// quad = quant chunk G, activations as scalar operands). The units of a phase
// are spread over every compute unit of the chip.
//
// Weights do not depend on activations, so the copies of phase p+1's columns
// into the LDS ring are issued as soon as phase p starts, right after its
// activation loads; they land while phase p computes and before phase p's
// end-of-phase synchronisation, whose loads and stores would otherwise queue
// behind them in the compute unit's memory pipeline (measured on MI355X: a
// phase handoff costs 2.8 us with idle compute units and 7 us while the same
// compute units stream).
//
// End of a phase: the quad's wavefront sums meet in LDS; a unit that covers a
// whole row stores y, one that covers part of it stores its partial sums
// (finished in split order at the end of the launch, or, for a matrix whose y
// is read by a later phase, by the tile's last unit at once, through a
// counter). Every wavefront then waits for its memory operations, the
// workgroup publishes its phase count in a flag, and before a dependent phase
// wavefront 0 polls all flags. Every wait is bounded: on a timeout the
// workgroup sets an error word and leaves, every poll sees the word and
// leaves too, and the host reads it (qwg_chain_status).
#include "qwg_device.h"
#include "q4k_dot.h"

namespace qwg {

namespace {

constexpr int kColBytes = kTileRows * kQ4kBytes;        // 9216
constexpr int kSlotBytes = kChainQuads * kColBytes;      // one step of the 4 quads
constexpr int kXOff = kChainRing * kSlotBytes;           // [wave][2 steps][64] fp32 activations
constexpr int kRedOff = kXOff + kChainQuads * 4 * 2 * 64 * 4;   // [quad][G][64] fp32
constexpr int kAbortOff = kRedOff + kChainQuads * 4 * 64 * 4;
constexpr int kLdsBytes = kAbortOff + 16;
static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");
static_assert(kChainMaxSteps * 2 <= kChainRing, "two phases' columns fit the ring");

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// A wait gives up after this many ticks of the 100 MHz constant clock (0.2 s):
// a whole chain normally takes well under a millisecond.
constexpr uint64_t kWaitTicks = 20000000;

__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stf_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Flags: one copy of all nwg flags per reader XCD (workgroup b runs on XCD
// b % 8), copies kFlagCopyWords apart; a workgroup stores its flag into every
// copy and polls the copy of its own XCD, so each copy's lines are read by
// the 32 workgroups of one XCD only. Within a copy the flags of the
// workgroups on one XCD share cache lines. Measured in a probe (flags only,
// idle chip): workgroup order 3.3 us per handoff, grouped by XCD 2.0 us,
// grouped and copied per reader XCD 1.86 us.
__device__ __forceinline__ int flag_pos(int b, int nwg) { return (b & 7) * (nwg >> 3) + (b >> 3); }
__device__ __forceinline__ uint32_t *flag_copy(const ChainArgs &c, int xcd) {
    return c.flags + xcd * kFlagCopyWords;
}

// True once every one of the nwg (<= 256) flags has reached `target`: one
// 16-byte agent-coherent load per lane.
__device__ __forceinline__ bool flags_reached(const uint32_t *flags, int nwg, uint32_t target) {
    const int lane = threadIdx.x & 63;
    bool ok = true;
    if (4 * lane < nwg) {
        u32x4_t f;
        asm volatile("global_load_dwordx4 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)"
                     : "=v"(f)
                     : "v"(flags + 4 * lane)
                     : "memory");
        ok = (int)(f[0] - target) >= 0 && (int)(f[1] - target) >= 0 && (int)(f[2] - target) >= 0 &&
             (int)(f[3] - target) >= 0;
    }
    return __builtin_amdgcn_ballot_w64(!ok) == 0;
}

// Wavefront 0: wait until every flag has reached `target`, or give up (the
// error word set by this or another workgroup, or the time bound). Returns
// false on giving up. One poll in flight at a time: the flag lines are read by
// every workgroup, and measured on MI355X, three polls in flight per
// workgroup slowed each round trip enough to lengthen the chain (473 -> 602
// us); the error word is read every 16th poll only (each read is another
// round trip).
__device__ bool wait_flags(const ChainArgs &c, uint32_t target, uint64_t t0) {
    const uint32_t *mine = flag_copy(c, blockIdx.x & 7);
    for (int i = 0;; ++i) {
        if (flags_reached(mine, c.nwg, target)) return true;
        if ((i & 15) == 15) {
            if (ld_agent(c.err) != 0u) return false;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
                if ((threadIdx.x & 63) == 0) st_agent(c.err, 1u);
                return false;
            }
        }
    }
}

// wait_vmcnt with a wavefront-uniform count of later copy instructions that
// may stay in flight (0, 3 or 6).
__device__ __forceinline__ void wait_vmcnt_n(int n) {
    switch (__builtin_amdgcn_readfirstlane(n)) {
        case 3: wait_vmcnt<3>(); break;
        case 6: wait_vmcnt<6>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

typedef const __attribute__((address_space(4))) ChainMember *cmember_p;

// A member descriptor read with scalar loads.
__device__ __forceinline__ void load_member(ChainMember &m, cmember_p p) {
    m.w = p->w;
    m.x = p->x;
    m.y = p->y;
    m.partial = p->partial;
    m.counters = p->counters;
    m.n_out = p->n_out;
    m.nb = p->nb;
    m.tiles = p->tiles;
    m.splits = p->splits;
    m.mode = p->mode;
}

// One quad's unit of a phase (its matrix's descriptor is read from the
// member table where needed: scalar loads that hit the scalar cache).
struct Unit {
    int member = -1;   // -1: no unit
    int tile = 0, b0 = 0, nblk = 0, split = 0;
};

__device__ __forceinline__ Unit load_unit(const ChainArgs &c, int phase, int col) {
    Unit u;
    if (phase >= c.nphases) return u;
    const cu32_p e = (cu32_p)c.units + ((size_t)phase * c.nwg * kChainQuads + col) * 4;
    const uint32_t mi = e[0];
    if (mi != kNoItem) {
        u.member = (int)mi;
        u.tile = (int)e[1];
        const uint32_t r = e[2];
        u.b0 = (int)(r & 0xFFu);
        u.nblk = (int)((r >> 8) & 0xFFu);
        u.split = (int)(r >> 16);
    }
    return u;
}

// The last unit of a tile to arrive sums the tile's partial sums in split
// order and stores its rows (agent-coherent: a later phase reads them), then
// re-arms the tile's counter. `t` is this unit's row sum (its partial).
__device__ void finish_tile_now(const ChainArgs &c, const Unit &u, float t) {
    const int lane = threadIdx.x & 63;
    ChainMember m;
    load_member(m, (cmember_p)c.members + u.member);
    const int row = u.tile * kTileRows + lane;
    const int64_t plane = (int64_t)m.tiles * kTileRows;
    stf_agent(&m.partial[(int64_t)u.split * plane + row], t);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    uint32_t old = 0;
    if (lane == 0)
        old = __hip_atomic_fetch_add(&m.counters[u.tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (uint32_t)(m.splits - 1)) return;
    float acc = 0.0f;
    for (int s0 = 0; s0 < m.splits; s0 += 8) {
        const float *pp[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            pp[k] = &m.partial[(int64_t)(s0 + k < m.splits ? s0 + k : s0) * plane + row];
        float v[8];
        load8_agent(pp, v);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (s0 + k < m.splits) acc += v[k];
    }
    if (row < m.n_out) stf_agent(&m.y[row], acc);
    if (lane == 0) st_agent(&m.counters[u.tile], 0u);
}

template <int G>
__device__ void chain_body(const ChainArgs &c, uint8_t *smem) {
    const int lane = threadIdx.x & 63;
    const int quad = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
    const int wave = 4 * quad + G;
    const int wg = blockIdx.x;
    const int col = wg * kChainQuads + quad;   // this quad's column of the unit table
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    volatile uint32_t *abort_word = (volatile uint32_t *)(smem + kAbortOff);
    float *red = (float *)(smem + kRedOff);
    const float *xl = (const float *)(smem + kXOff) + wave * 2 * 64;   // this wavefront's activations
    const uint32_t xbase = lds0 + kXOff + wave * 2 * 64 * 4;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();

    // Every workgroup's flag holds the same count at the start (every earlier
    // run completed all its phases).
    uint32_t base = 0;
    if (wave == 0) base = ld_agent(&flag_copy(c, wg & 7)[flag_pos(wg, c.nwg)]);

    // Copies of a unit's columns into ring slots slot0, slot0 + 1, ...: the
    // quad's wavefronts 1..3 move bytes 3072(G-1) .. 3072G - 1 of each
    // 9216-byte column (three instructions of 64 lanes x 16 bytes). Wavefront
    // 0, which stores the quad's sums at the end of a phase, copies no
    // weights, so that its wait for those stores does not also wait for the
    // next phase's columns. Returns the number of copy instructions issued.
    const uint32_t coff = 3072 * (G > 0 ? G - 1 : 0) + 16 * lane;
    auto issue_unit = [&](const Unit &u, int slot0) {
        if (G == 0 || u.member < 0) return 0;
        const cmember_p mp = (cmember_p)c.members + u.member;
        const uint8_t *colp = mp->w + ((int64_t)u.tile * mp->nb + u.b0) * kColBytes + coff;
        for (int s = 0; s < u.nblk; ++s) {
            const uint32_t dst = lds0 + ((slot0 + s) & (kChainRing - 1)) * kSlotBytes +
                                 quad * kColBytes + 3072 * (G - 1);
            const uint8_t *src = colp + (int64_t)s * kColBytes;
            dma16_stream(src, dst);
            dma16_stream(src + 1024, dst + 1024);
            dma16_stream(src + 2048, dst + 2048);
        }
        return 3 * u.nblk;
    };

    const uint32_t mlo = opaque(0x000F000Fu);
    const uint32_t mhi = opaque(0x00F000F0u);
    int step = 0;   // ring slot of the current phase's first column
    Unit u = load_unit(c, 0, col);
    issue_unit(u, 0);
    Unit un = load_unit(c, 1, col);
    bool aborted = false;
    for (int p = 0; p < c.nphases; ++p) {
        // This phase's activations (their producers are complete): the 64 of
        // each of the unit's columns for this wavefront's quant chunk, copied
        // into LDS ahead of the next phase's weight columns.
        const cmember_p mp = (cmember_p)c.members + (u.member >= 0 ? u.member : 0);
        if (u.member >= 0 && lane < 16) {
            const float *xg = mp->x + (int64_t)kQK * u.b0 + 64 * G + 4 * lane;
            const uint32_t xd = lds0 + kXOff + wave * 2 * 64 * 4;
            for (int s = 0; s < u.nblk; ++s) dma16(xg + kQK * s, xd + 256 * s);
        }
        // The next phase's columns (weights do not depend on activations).
        const int newer = issue_unit(un, step + (int)((cu32_p)c.phases)[2 * p]);
        // This phase's columns (issued one phase ago) and its activations are
        // older than the copies just issued.
        wait_vmcnt_n(newer);
        lds_barrier();
        float acc = 0.0f;
        if (u.member >= 0) {
            for (int s = 0; s < u.nblk; ++s) {
                const int slot = (step + s) & (kChainRing - 1);
                const uint8_t *rowp = smem + slot * kSlotBytes + quad * kColBytes + lane * kQ4kBytes;
                const float hs = half_wave_sum(xl[64 * s + lane]);
                const float sx0 = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hs), 16));
                const float sx1 = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, hs), 48));
                // The activations as operands: the same LDS copy, read at one
                // address by every lane (broadcast), instead of a second round
                // trip of scalar loads after the copy has landed.
                const uint32_t xa = xbase + 256 * s;
                f32x4 xv[16];
#pragma unroll
                for (int k = 0; k < 16; ++k) xv[k] = lds_load<f32x4>(xa + 16 * k);
                q4k_chunk_2chains<G>(
                    rowp, [&](int i) { return xv[i >> 2][i & 3]; }, sx0, sx1, mlo, mhi, acc);
            }
        }
        // Row sums of the quad's four wavefronts, in wavefront order.
        red[wave * 64 + lane] = acc;
        lds_barrier();
        if (G == 0 && u.member >= 0) {
            float t = red[(4 * quad) * 64 + lane];
#pragma unroll
            for (int g = 1; g < 4; ++g) t += red[(4 * quad + g) * 64 + lane];
            const int row = u.tile * kTileRows + lane;
            if (mp->splits == 1) {
                if (row < mp->n_out) stf_agent(&mp->y[row], t);
            } else if (mp->mode == kChainDeferred) {
                stf_agent(&mp->partial[(int64_t)u.split * mp->tiles * kTileRows + row], t);
            } else {
                finish_tile_now(c, u, t);
            }
        }
        // The unit after next: its descriptor loads overlap the wait below.
        const int Lp = (int)((cu32_p)c.phases)[2 * p];
        Unit unn = load_unit(c, p + 2, col);
        // Every store of this phase has completed before the workgroup counts
        // the phase as done (the stores are wavefront 0's of each quad; the
        // next phase's columns may still be in flight).
        if (G == 0) wait_vmcnt<0>();
        lds_barrier();
        if (wave == 0) {
            if (lane < kFlagCopies)
                st_agent(&flag_copy(c, lane)[flag_pos(wg, c.nwg)], base + (uint32_t)p + 1u);
            const bool wait_next = p + 1 < c.nphases && ((cu32_p)c.phases)[2 * (p + 1) + 1] != 0u;
            const bool last = p + 1 == c.nphases && c.nfin > 0;
            if ((wait_next || last) && !wait_flags(c, base + (uint32_t)p + 1u, t0)) *abort_word = 1u;
        }
        lds_barrier();
        // (read as a wave-uniform value, so that the loop stays scalar)
        if (__builtin_amdgcn_readfirstlane(*abort_word) != 0u) {
            aborted = true;
            break;
        }
        step += Lp;
        u = un;
        un = unn;
    }
    if (aborted) {
        wait_vmcnt<0>();
        return;
    }
    // Partial sums of the deferred matrices (every phase is complete): each
    // tile's partials summed in split order, its rows stored.
    const int waves_total = c.nwg * kChainQuads * 4;
    for (int f = wg * kChainQuads * 4 + wave; f < c.nfin; f += waves_total) {
        const uint32_t mi = ((cu32_p)c.fin)[2 * f];
        const int tile = (int)((cu32_p)c.fin)[2 * f + 1];
        ChainMember fm;
        load_member(fm, (cmember_p)c.members + mi);
        const int row = tile * kTileRows + lane;
        const int64_t plane = (int64_t)fm.tiles * kTileRows;
        float t = 0.0f;
        for (int s0 = 0; s0 < fm.splits; s0 += 8) {
            const float *pp[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                pp[k] = &fm.partial[(int64_t)(s0 + k < fm.splits ? s0 + k : s0) * plane + row];
            float v[8];
            load8_agent(pp, v);
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (s0 + k < fm.splits) t += v[k];
        }
        if (row < fm.n_out) fm.y[row] = t;
    }
}

__global__ __launch_bounds__(kChainQuads * 256) void q4k_chain_kernel(ChainArgs c) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    if (threadIdx.x == 0) *(volatile uint32_t *)(smem + kAbortOff) = 0u;
    __syncthreads();
    switch (__builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3)) {
        case 0: chain_body<0>(c, smem); break;
        case 1: chain_body<1>(c, smem); break;
        case 2: chain_body<2>(c, smem); break;
        default: chain_body<3>(c, smem); break;
    }
}

}  // namespace

int chain_lds_bytes() { return kLdsBytes; }

hipError_t launch_q4k_chain(const ChainArgs &c, hipStream_t s) {
    if (c.nwg < 8 || c.nwg > 256 || c.nwg % 8) return hipErrorInvalidValue;
    hipLaunchKernelGGL(q4k_chain_kernel, dim3((unsigned)c.nwg), dim3(kChainQuads * 256), kLdsBytes,
                       s, c);
    return hipGetLastError();
}

}  // namespace qwg
