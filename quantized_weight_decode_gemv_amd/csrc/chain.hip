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
// One workgroup per compute unit, 16 wavefronts = 4 quads. Per phase a
// workgroup takes one chunk of one 64-row tile of one matrix: up to eight
// super-block columns (tile layout: a column is 9216 contiguous bytes), two
// per quad; each quad computes its columns as the GEMV engines do (lane =
// row, wavefront G of the quad = quant chunk G, activations as operands from
// LDS), and the sixteen wavefronts' row sums meet in LDS. A row of up to eight
// columns (n_in <= 2048) is thus finished by one workgroup without a trip
// through memory; a longer row is cut into chunks whose partial sums meet
// through memory. The tile chunks of a phase are spread over the workgroups.
//
// Weights do not depend on activations, so the copies of phase p+1's columns
// into the LDS ring are issued as soon as phase p starts, right after its
// activation loads; they land while phase p computes and before phase p's
// end-of-phase synchronisation, whose loads and stores would otherwise queue
// behind them in the compute unit's memory pipeline (measured on MI355X: a
// phase handoff costs 2.8 us with idle compute units and 7 us while the same
// compute units stream).
//
// End of a phase: the workgroup's wavefront sums meet in LDS; a unit that covers a
// whole row stores y, one that covers part of it stores its partial sums
// (finished in split order at the end of the launch, or, for a matrix whose y
// is read by a later phase, by the tile's last unit at once, through a
// counter). A phase starts only once every tile of the phase before it is
// finished (a decode step's norms and attention need all of their producer's
// rows), in one of two ways:
//  * tagged (when every activation read from the chain lies inside one earlier
//    member's output and no output overlaps another output or an earlier
//    phase's activations): the unit that finishes a tile stores a done word,
//    the tile's sum of squares of y (the datum an rmsnorm between the phases
//    needs from every row) | tag << 32, in one 8-byte store; a member whose y
//    a later member reads also stores each row so tagged. Wavefront 0 of a
//    workgroup loads the previous phase's done words until every tag is this
//    run's; wavefront 0 of a quad loads its unit's tagged activations the same
//    way and places them in LDS. Readiness and data arrive in one round trip,
//    no store waits for an earlier one to complete, and a phase waits for its
//    producers' tiles, not for every workgroup's stores. One flag barrier
//    remains, after the last phase, for the matrices finished there.
//  * barrier: every wavefront waits for its memory operations, the workgroup
//    publishes its phase count in a flag, and before a dependent phase
//    wavefront 0 polls all flags.
// Every wait is bounded: on a timeout the workgroup sets an error word and
// leaves, every poll sees the word and leaves too, and the host reads it
// (qwg_chain_status).
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
// A tagged row: one single-copy-atomic 8-byte store, so a reader sees the value
// and its tag together.
__device__ __forceinline__ void st_tagged(uint64_t *p, float v, uint32_t tag) {
    __hip_atomic_store(p, (uint64_t)__builtin_bit_cast(uint32_t, v) | ((uint64_t)tag << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Eight agent-coherent 8-byte loads issued back to back, one wait for all.
__device__ __forceinline__ void load8_tagged(const uint64_t *const (&p)[8], uint64_t (&v)[8]) {
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

// Two, three or four agent-coherent 8-byte loads back to back, one wait.
__device__ __forceinline__ void load2_tagged(const uint64_t *p0, const uint64_t *p1, uint64_t &v0,
                                             uint64_t &v1) {
    asm volatile(
        "global_load_dwordx2 %0, %2, off sc1\n\t"
        "global_load_dwordx2 %1, %3, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v0), "=&v"(v1)
        : "v"(p0), "v"(p1)
        : "memory");
}
__device__ __forceinline__ void load3_tagged(const uint64_t *p0, const uint64_t *p1,
                                             const uint64_t *p2, uint64_t &v0, uint64_t &v1,
                                             uint64_t &v2) {
    asm volatile(
        "global_load_dwordx2 %0, %3, off sc1\n\t"
        "global_load_dwordx2 %1, %4, off sc1\n\t"
        "global_load_dwordx2 %2, %5, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2)
        : "v"(p0), "v"(p1), "v"(p2)
        : "memory");
}
__device__ __forceinline__ void load4_tagged(const uint64_t *const (&p)[4], uint64_t (&v)[4]) {
    asm volatile(
        "global_load_dwordx2 %0, %4, off sc1\n\t"
        "global_load_dwordx2 %1, %5, off sc1\n\t"
        "global_load_dwordx2 %2, %6, off sc1\n\t"
        "global_load_dwordx2 %3, %7, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
        : "memory");
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

// Tagged, wavefront 0 of a workgroup: wait until the n done words at `done`
// all carry a tag at or past `tag`. Bounded as wait_flags.
__device__ bool wait_done(const ChainArgs &c, const uint64_t *done, int n, uint32_t tag,
                          uint64_t t0) {
    const int lane = threadIdx.x & 63;
    for (int i = 0;; ++i) {
        bool ok = true;
        for (int j0 = 0; j0 < n; j0 += 512) {
            // up to eight 8-byte loads per lane (64 words each) in flight, one
            // wait; rounds of fewer words load fewer
            const int m = min(n - j0, 512);
            // as many loads as the round has 64-word groups (no repeated
            // reads of the last word: every workgroup polls these lines)
            if (m <= 64) {
                uint64_t v;
                asm volatile("global_load_dwordx2 %0, %1, off sc1\n\ts_waitcnt vmcnt(0)"
                             : "=v"(v)
                             : "v"(done + j0 + min(lane, m - 1))
                             : "memory");
                ok = ok && (int)((uint32_t)(v >> 32) - tag) >= 0;
            } else if (m <= 128) {
                uint64_t v0, v1;
                load2_tagged(done + j0 + lane, done + j0 + min(64 + lane, m - 1), v0, v1);
                ok = ok && (int)((uint32_t)(v0 >> 32) - tag) >= 0 &&
                     (int)((uint32_t)(v1 >> 32) - tag) >= 0;
            } else if (m <= 192) {
                uint64_t v0, v1, v2;
                load3_tagged(done + j0 + lane, done + j0 + 64 + lane,
                             done + j0 + min(128 + lane, m - 1), v0, v1, v2);
                ok = ok && (int)((uint32_t)(v0 >> 32) - tag) >= 0 &&
                     (int)((uint32_t)(v1 >> 32) - tag) >= 0 &&
                     (int)((uint32_t)(v2 >> 32) - tag) >= 0;
            } else if (m <= 256) {
                const uint64_t *p[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) p[k] = done + j0 + min(64 * k + lane, m - 1);
                uint64_t v[4];
                load4_tagged(p, v);
#pragma unroll
                for (int k = 0; k < 4; ++k) ok = ok && (int)((uint32_t)(v[k] >> 32) - tag) >= 0;
            } else {
                const uint64_t *p[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) p[k] = done + j0 + min(64 * k + lane, m - 1);
                uint64_t v[8];
                load8_tagged(p, v);
#pragma unroll
                for (int k = 0; k < 8; ++k) ok = ok && (int)((uint32_t)(v[k] >> 32) - tag) >= 0;
            }
        }
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) return true;
        if ((i & 15) == 15) {
            if (ld_agent(c.err) != 0u) return false;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
                if (lane == 0) st_agent(c.err, 1u);
                return false;
            }
        }
    }
}

// Sum over the wavefront, wave-uniform: the two half-wave sums of the DPP
// reduction (lanes 16 and 48), added in that order.
__device__ __forceinline__ float wave_sum(float v) {
    const int h = __builtin_bit_cast(int, half_wave_sum(v));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(h, 16)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(h, 48));
}

// The done word of a (tile, split) (tagged launches): the sum of squares of
// its rows (of y, or of the split's partial sums).
__device__ __forceinline__ void store_done(const ChainMember &m, int tile, int split, float y,
                                           bool valid, uint32_t base) {
    const float ss = wave_sum(valid ? y * y : 0.0f);
    if ((threadIdx.x & 63) == 0)
        st_tagged(&m.done[(int64_t)tile * m.splits + split], ss, base + (uint32_t)m.tag);
}

// Tagged, wavefront 0 of a quad: wait until the unit's activations all carry
// a tag at or past `tag`, then put them into the four wavefronts' LDS
// activation slots (wavefront g of the quad: k = 64g .. 64g + 63 of column s,
// at xq + 128 g + 64 s). Activation k of the unit's column s is the sum, in
// split order, of the producer's nsp partials xll[sp * stride + 256 (b0 + s)
// + k]. The loads go out eight at a time (one wait per eight).
// This wavefront copies no weights, so its waits wait for nothing else.
// Bounded as wait_flags; returns false on giving up.
__device__ __forceinline__ bool wait_x(const ChainArgs &c, const uint64_t *xll, int nsp,
                                       int stride, int b0, int nblk, uint32_t tag, float *xq,
                                       uint64_t t0) {
    const int lane = threadIdx.x & 63;
    // Eight loads per round: two columns of one split (nblk = 2), or one
    // column of two splits (nblk = 1; an odd last round loads its split twice
    // and adds it once). Slot j: wavefront g = j & 3.
    const int per = nblk == 2 ? 1 : 2;   // splits per round
    for (int i = 0;; ++i) {
        float sum[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};   // [s][g]
        bool ok = true;
        for (int sp0 = 0; sp0 < nsp; sp0 += per) {
            const uint64_t *p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int s = nblk == 2 ? (j >> 2) : 0;
                const int sp = nblk == 2 ? sp0 : min(sp0 + (j >> 2), nsp - 1);
                p[j] = xll + (int64_t)sp * stride + 256 * (b0 + s) + 64 * (j & 3) + lane;
            }
            uint64_t v[8];
            load8_tagged(p, v);
            const bool second = nblk == 2 || sp0 + 1 < nsp;   // slots 4..7 hold new values
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < 4 || second) {
                    ok = ok && (int)((uint32_t)(v[j] >> 32) - tag) >= 0;
                    // nblk = 1: slot j + 4 is the next split of the same k
                    sum[nblk == 2 ? j : (j & 3)] += __builtin_bit_cast(float, (uint32_t)v[j]);
                }
            }
        }
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if ((k >> 2) < nblk) xq[128 * (k & 3) + 64 * (k >> 2) + lane] = sum[k];
            return true;
        }
        if ((i & 15) == 15) {
            if (ld_agent(c.err) != 0u) return false;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
                if (lane == 0) st_agent(c.err, 1u);
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
    m.ll = p->ll;
    m.xll = p->xll;
    m.done = p->done;
    m.xsplits = p->xsplits;
    m.xstride = p->xstride;
    m.tag = p->tag;
    m.xtag = p->xtag;
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
__device__ void finish_tile_now(const ChainArgs &c, const Unit &u, float t, uint32_t base) {
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
    if (row < m.n_out) {
        stf_agent(&m.y[row], acc);
        if (m.ll) st_tagged(&m.ll[row], acc, base + (uint32_t)m.tag);
    }
    if (c.tagged && m.done) store_done(m, u.tile, 0, acc, row < m.n_out, base);
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
    // The abort word through an LDS pointer: as a generic pointer it became a
    // flat load, after which the compiler waits for every outstanding memory
    // operation, this wavefront's copies of the next phase's columns included.
    volatile __attribute__((address_space(3))) uint32_t *abort_word =
        (volatile __attribute__((address_space(3))) uint32_t *)(size_t)(lds0 + kAbortOff);
    float *red = (float *)(smem + kRedOff);
    const float *xl = (const float *)(smem + kXOff) + wave * 2 * 64;   // this wavefront's activations
    const uint32_t xbase = lds0 + kXOff + wave * 2 * 64 * 4;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();

    // Every workgroup's flag holds the same count at the start (every earlier
    // run completed all its phases); it is this run's base of phase counts and
    // tags.
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        ld_agent(&flag_copy(c, wg & 7)[flag_pos(wg, c.nwg)]));

    // Copies of a unit's columns into ring slots slot0, slot0 + 1, ...: the
    // quad's wavefronts 1..3 move bytes 3072(G-1) .. 3072G - 1 of each
    // 9216-byte column (three instructions of 64 lanes x 16 bytes). The quads'
    // wavefronts 0 copy no weights: the workgroup's wavefront 0 stores the
    // sums at the end of a phase and loads the done words, and each quad's
    // wavefront 0 loads its unit's tagged activations, so their waits for
    // those loads and stores wait for nothing else (per-wavefront memory
    // counters complete in order). Returns the number of copy instructions
    // issued.
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
        const uint64_t *xll = u.member >= 0 && c.tagged ? mp->xll : nullptr;
        if (xll != nullptr) {
            if (G == 0 && !wait_x(c, xll, mp->xsplits, mp->xstride, u.b0, u.nblk,
                                  base + (uint32_t)mp->xtag,
                                  (float *)(smem + kXOff) + 4 * quad * 2 * 64, t0))
                *abort_word = 1u;
        } else if (u.member >= 0 && lane < 16) {
            const float *xg = mp->x + (int64_t)kQK * u.b0 + 64 * G + 4 * lane;
            const uint32_t xd = lds0 + kXOff + wave * 2 * 64 * 4;
            for (int s = 0; s < u.nblk; ++s) dma16(xg + kQK * s, xd + 256 * s);
        }
        // Tagged launches: the previous phase's tiles are all finished (wave
        // 0's loads queue behind no weight copies of its own).
        if (c.tagged && wave == 0 && u.member >= 0) {   // (quad 0 holds the workgroup's chunk)
            const cu32_p ph = (cu32_p)c.phases + 4 * p;
            const int nd = (int)ph[2];
            if (nd > 0 && !wait_done(c, c.done + ph[3], nd, base + ph[1], t0)) *abort_word = 1u;
        }
        // The next phase's columns (weights do not depend on activations).
        const int newer = issue_unit(un, step + (int)((cu32_p)c.phases)[4 * p]);
        // This phase's columns (issued one phase ago) and its activations are
        // older than the copies just issued.
        wait_vmcnt_n(newer);
        lds_barrier();
        if (c.tagged && __builtin_amdgcn_readfirstlane(*abort_word) != 0u) {
            aborted = true;
            break;
        }
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
        // Row sums of the workgroup's sixteen wavefronts (its quads hold column
        // pairs of one tile chunk; a quad without columns adds zeros), in
        // wavefront order.
        red[wave * 64 + lane] = acc;
        lds_barrier();
        if (wave == 0 && u.member >= 0) {
            float t = red[lane];
#pragma unroll
            for (int w = 1; w < kChainQuads * 4; ++w) t += red[w * 64 + lane];
            const int row = u.tile * kTileRows + lane;
            if (mp->splits == 1) {
                if (row < mp->n_out) {
                    stf_agent(&mp->y[row], t);
                    if (c.tagged && mp->ll) st_tagged(&mp->ll[row], t, base + (uint32_t)mp->tag);
                }
                if (c.tagged && mp->done) {
                    ChainMember m;
                    load_member(m, mp);
                    store_done(m, u.tile, 0, t, row < mp->n_out, base);
                }
            } else if (mp->mode == kChainDeferred) {
                // tagged launches: a consumed member's partials are its tagged rows
                if (c.tagged && mp->ll) {
                    if (row < mp->n_out)
                        st_tagged(&mp->ll[(int64_t)u.split * mp->n_out + row], t,
                                  base + (uint32_t)mp->tag);
                } else {
                    stf_agent(&mp->partial[(int64_t)u.split * mp->tiles * kTileRows + row], t);
                }
                if (c.tagged && mp->done) {
                    ChainMember m;
                    load_member(m, mp);
                    store_done(m, u.tile, u.split, t, row < mp->n_out, base);
                }
            } else {
                finish_tile_now(c, u, t, base);
            }
        }
        // The unit after next: its descriptor loads overlap the wait below.
        const int Lp = (int)((cu32_p)c.phases)[4 * p];
        Unit unn = load_unit(c, p + 2, col);
        if (c.tagged && p + 1 < c.nphases) {
            // no end-of-phase barrier: the next phase waits for the done words
            step += Lp;
            u = un;
            un = unn;
            continue;
        }
        // Every store of this phase has completed before the workgroup counts
        // the phase as done (the stores are wavefront 0's; the
        // next phase's columns may still be in flight).
        if (G == 0) wait_vmcnt<0>();
        lds_barrier();
        if (wave == 0) {
            if (lane < kFlagCopies)
                st_agent(&flag_copy(c, lane)[flag_pos(wg, c.nwg)], base + (uint32_t)p + 1u);
            const bool wait_next = p + 1 < c.nphases && ((cu32_p)c.phases)[4 * (p + 1) + 1] != 0u;
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
        if (c.tagged && fm.ll) {   // partials as tagged rows [splits][n_out]
            const int r = min(row, fm.n_out - 1);
            for (int s0 = 0; s0 < fm.splits; s0 += 8) {
                const uint64_t *pp[8];
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    pp[k] = &fm.ll[(int64_t)(s0 + k < fm.splits ? s0 + k : s0) * fm.n_out + r];
                uint64_t v[8];
                load8_tagged(pp, v);
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (s0 + k < fm.splits) t += __builtin_bit_cast(float, (uint32_t)v[k]);
            }
            if (row < fm.n_out) fm.y[row] = t;
            continue;
        }
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
    if (threadIdx.x == 0)
        *(volatile __attribute__((address_space(3))) uint32_t *)(size_t)((uint32_t)(uintptr_t)smem +
                                                                        kAbortOff) = 0u;
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
