// C ABI of libqwg (declared in include/qwg.h): argument validation, work
// decomposition and launch. Every check runs on the host before any HIP call,
// so a rejected call touches neither the device nor the output buffers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>
#include <map>
#include <mutex>
#include <queue>
#include <utility>

#include "../../include/qwg.h"
#include "qwg_internal.h"
#include "short_call.h"

using namespace qwg;

namespace {

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_gemv_shape(int64_t n_in, int64_t n_out) {
    if (n_in < kQK || n_in > QWG_MAX_N_IN || n_in % kQK) return QWG_ERR_SHAPE;
    if (n_out < 1 || n_out > QWG_MAX_N_OUT) return QWG_ERR_SHAPE;
    return QWG_OK;
}

int env_int(const char *name, int dflt) {
    const char *e = getenv(name);
    const int v = e ? atoi(e) : 0;
    return v > 0 ? v : dflt;
}

// Work decomposition of one GEMV/GEMM: W wavefronts per 64-row tile (W/4
// super-blocks per pipeline stage) and the number of workgroups that split each
// tile's super-block range. Matrices with many tiles use 16-wavefront groups
// and no split; small ones use 4-wavefront groups and split the row sums so the
// grid still covers every compute unit (about kSplitTargetWgs workgroups).
// QWG_WAVES / QWG_TARGET_WGS override the choice (tuning experiments).
constexpr int kLargeTiles = 256;
constexpr int kSplitTargetWgs = 2048;
constexpr size_t kWsPartialFloats = (size_t)2 * kSplitTargetWgs * QWG_MAX_BATCH * kTileRows;
constexpr size_t kWsCounters = 2 * kSplitTargetWgs;

struct Plan {
    int waves;
    int splits;
};

Plan choose_plan(int tiles, int nb, int batch) {
    static const int env_waves = env_int("QWG_WAVES", 0);
    static const int env_target = env_int("QWG_TARGET_WGS", 0);
    Plan p;
    p.waves = env_waves ? env_waves : (tiles >= kLargeTiles ? kQ4kWavesLarge : kQ4kWavesSmall);
    if (p.waves != 4 && p.waves != 8 && p.waves != 16) p.waves = kQ4kWavesSmall;
    const int target = env_target ? env_target : (tiles >= kLargeTiles ? 1 : kSplitTargetWgs);
    int s = (target + tiles - 1) / tiles;
    if (s > nb) s = nb;
    if (s < 1) s = 1;
    // keep the partial sums inside the workspace
    while (s > 1 && ((size_t)s * batch * tiles * kTileRows > kWsPartialFloats ||
                     (size_t)tiles > kWsCounters))
        --s;
    p.splits = s;
    return p;
}

int choose_splits(int tiles, int nb) { return choose_plan(tiles, nb, 1).splits; }

// Splits of a matrix-core GEMM (batch >= 2): at least kMfmaTargetWgs
// workgroups, at most one split per super-block, partial sums inside the
// workspace. Each workgroup's few stages are latency-bound, so a short launch
// wants enough workgroups to overlap them but not so many that every one does
// a single stage. Measured at batch 8 (us, by splits): 2048 x 2048 (32 tiles)
// 1: 10.9, 2: 9.2, 4: 8.5, 8: 9.9; 5632 x 2048 (88 tiles) 1: 11.1, 2: 9.5,
// 4: 9.9; the 32000 x 2048 LM head (500 tiles) 1: 15.5, 2: 17.2.
// QWG_MFMA_TARGET overrides the target (tuning).
constexpr int kMfmaTargetWgs = 128;

int mfma_splits(int tiles, int nb, int batch) {
    static const int env_target = env_int("QWG_MFMA_TARGET", 0);
    const int target = env_target ? env_target : kMfmaTargetWgs;
    int s = (target + tiles - 1) / tiles;
    if (s > nb) s = nb;
    if (s < 1) s = 1;
    while (s > 1 && ((size_t)s * batch * tiles * kTileRows > kWsPartialFloats ||
                     (size_t)tiles > kWsCounters))
        --s;
    return s;
}

// Batch-2 GEMMs of at least this many 64-row tiles run on the vector ALUs.
constexpr int kValuBatch2Tiles = 256;

// waves arguments of qwg_gemm_q4k_ex that select the matrix-core engines: the
// one-workgroup-per-tile pipeline with one or two super-block columns per
// stage, or the persistent batched stream
constexpr int kWavesMfma = 1;
constexpr int kWavesMfma2 = 2;
constexpr int kWavesMstream = 3;

// Batch 2..8 runs on the one-workgroup-per-tile pipeline (q4k_mfma_kernel /
// q4k_mfma_group_kernel) unless QWG_MFMA_ENGINE=1 selects the persistent
// batched stream (q4k_mstream_kernel) for every call and group (A/B tuning).
// Measured A/B (cold weights, us, per-tile pipeline / persistent stream): LM
// head 32000 x 2048 at batch 8 15.1-16.7 / 15.8 (whole rows, 2-stage ring;
// 17-33 with split rows); 5632 x 2048 9.3-9.6 / 9.5-11; 2048 x 5632 11.6 /
// 11.2-24 (by splits); the 155-product batched stream at batch 8 180 / 192.
// The stream's ring hides no more than the pipeline already does: each stage
// is a long chain of dependent LDS, MFMA and ALU steps, and both engines issue
// the same 27 MFMAs and ~200-260 vector instructions per stage and wavefront.
bool mfma_tile_engine() {
    static const int v = env_int("QWG_MFMA_ENGINE", 0);
    return v != 1;
}

// Ring stages of the batched stream (QWG_MSTREAM_RING overrides, tuning):
// two, measured best (more workgroups per CU; LM head at batch 8 15.8 us with
// two stages, 17.0 with three, 17.7 with four).
int mstream_ring() {
    static const int v = [] {
        const int r = env_int("QWG_MSTREAM_RING", 2);
        return r >= 2 && r <= 4 ? r : 2;
    }();
    return v;
}

// Splits of a single batched-stream GEMM: about one item per compute unit
// (split rows end in an epilogue round trip per item), at most one split per
// super-block, partial sums inside the workspace. Measured (us, by splits):
// LM head (500 tiles) 1: 15.8, 2: 17.9; 5632 x 2048 (88 tiles) 1: 11.1, 2-4:
// 9.7; 2048 x 5632 (32 tiles) 1: 24.1, 4: 11.8, 6: 11.2 (QWG_MSTREAM_SPLITS
// overrides, tuning).
int mstream_splits(int tiles, int nb, int batch, int slots) {
    static const int env = env_int("QWG_MSTREAM_SPLITS", 0);
    (void)slots;
    int s = env > 0 ? env : (256 + tiles - 1) / tiles;
    if (s > nb) s = nb;
    if (s < 1) s = 1;
    while (s > 1 && ((size_t)s * batch * tiles * kTileRows > kWsPartialFloats ||
                     (size_t)tiles > kWsCounters))
        --s;
    return s;
}

// Ring stages of the matrix-core engine. Measured (LM head, batch 8, one
// split): 2 stages 17.0 us, 3 stages 17.6 us, 4 stages 18.5 us; deeper rings
// only cost occupancy. QWG_MFMA_RING overrides it (tuning).
int mfma_ring() {
    static const int v = [] {
        const int r = env_int("QWG_MFMA_RING", 2);
        return r >= 2 && r <= 4 ? r : 2;
    }();
    return v;
}

// Columns per stage of the matrix-core engine (cols 0 = automatic): two (8
// wavefronts per tile) when every workgroup's range has at least two
// super-blocks and either the batch is small or the launch has few
// workgroups, else one. Measured: LM head batch 2: 15.5 -> 14.7 us, batch 8:
// 15.5 -> 16.3 us (500 workgroups); 5632 x 2048 at 2 splits, batch 2: 9.3 ->
// 8.3 us, batch 8: 9.7 -> 9.5 us. QWG_MFMA_COLS forces 1 or 2 for the
// automatic choice (tuning). Two columns run with a 2-stage ring (deeper
// rings leave one workgroup per CU).
hipError_t launch_mfma(const GemvArgs &a, int batch, hipStream_t s, int cols = 0,
                       bool tiled = false) {
    static const int env_cols = env_int("QWG_MFMA_COLS", 0);
    if (cols == 0) {
        const bool two = a.nb / a.splits >= 2 && (batch <= 4 || a.tiles * a.splits <= 256);
        cols = two ? 2 : 1;
        if (env_cols == 1 || env_cols == 2) cols = env_cols;
    }
    const int ring = cols == 2 || tiled ? 2 : mfma_ring();
    return launch_q4k_mfma(a, batch, ring, cols, tiled, s);
}

// Persistent stream engine shape (wavefronts per workgroup, LDS ring stages).
// Measured on MI355X: grouped streams run best with 4-wavefront workgroups and
// a 2-stage ring (more resident workgroups per CU); a single large matrix, with
// fewer tiles than workgroup slots, with 8 wavefronts per tile.
// QWG_STREAM_WAVES / QWG_STREAM_RING override both (tuning experiments).
struct StreamShape {
    int waves;
    int ring;
};

StreamShape stream_shape(bool grouped) {
    static const int env_w = env_int("QWG_STREAM_WAVES", 0);
    static const int env_r = env_int("QWG_STREAM_RING", 0);
    StreamShape sh;
    sh.waves = env_w ? env_w : (grouped ? 4 : 8);
    sh.ring = env_r ? env_r : 2;
    const bool built = (sh.waves == 4 || sh.waves == 8 || sh.waves == 16) &&
                       (sh.ring == 2 || sh.ring == 3);
    if (!built) sh = {grouped ? 4 : 8, 2};  // an override with no compiled variant
    return sh;
}

bool stream_shape_overridden() {
    static const bool v = env_int("QWG_STREAM_WAVES", 0) != 0 || env_int("QWG_STREAM_RING", 0) != 0;
    return v;
}

bool use_stream_engine() {
    static const bool v = env_int("QWG_TILE_ENGINE", 0) == 0;
    return v;
}

// Compute units of the current device (0 on error), cached per device.
int device_cus() {
    static std::mutex mu;
    static std::map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    cache.emplace(dev, cus);
    return cus;
}

// Splits of a batch-1 Q4_K or IQ3 call on the short-call kernels, or 0 for the
// other engines: matrices whose tiles x splits fit one workgroup per compute
// unit.
// QWG_SHORT=0 turns the short-call kernel off (A/B measurements).
int short_splits(int tiles, int nb) {
    static const bool off = [] {
        const char *e = getenv("QWG_SHORT");
        return e != nullptr && e[0] == '0';
    }();
    if (off) return 0;
    const int cus = device_cus();
    const int sp = cus > 0 ? short_plan_splits(tiles, nb, cus) : 0;
    // QWG_SHORT_SPLITS caps the splits (tuning experiments)
    static const int cap = env_int("QWG_SHORT_SPLITS", 0);
    if (sp > 0 && cap > 0 && sp > cap) {
        if ((nb + cap - 1) / cap > kShortMaxBlocks) return sp;
        return cap;
    }
    return sp;
}

// Batch-1 Q4_K, IQ3, IQ3_S and IQ4_XS calls on the row-group kernels: the
// short-call matrices whose rows hold at most 8 (Q4_K) or 24 (the others)
// blocks. (Not larger matrices: the Q4_K LM
// head, 32000 x 2048, took 17.4 us per call on row groups against 11.0 us on
// the stream engine, event time on one box.) QWG_ROWS=0 turns them off (A/B
// measurements: those matrices then run on the split short-call kernels).
bool rows_off() {
    static const bool off = [] {
        const char *e = getenv("QWG_ROWS");
        return e != nullptr && e[0] == '0';
    }();
    return off;
}
bool rows_engine(int tiles, int nb) {
    return !rows_off() && q4k_rows_fits(nb) && short_splits(tiles, nb) > 0;
}
bool rows_engine_iq3(int tiles, int nb) {
    return !rows_off() && iq3_rows_fits(nb) && short_splits(tiles, nb) > 0;
}
bool rows_engine_cb(int tiles, int nb) {
    return !rows_off() && cb_rows_fits(nb) && short_splits(tiles, nb) > 0;
}

// IQ3 stream engine shape. Measured on MI355X: grouped streams run best with
// 8-wavefront workgroups (two per CU), single GEMVs with 16 (one per CU, four
// super-blocks per stage), both with a 2-stage ring. `waves` (if nonzero)
// overrides the wavefront count; QWG_IQ3_WAVES / QWG_IQ3_RING override both
// (tuning experiments). An unsupported combination falls back to the default.
Iq3Shape iq3_shape(bool grouped, int waves) {
    static const int env_w = env_int("QWG_IQ3_WAVES", 0);
    static const int env_r = env_int("QWG_IQ3_RING", 0);
    const Iq3Shape dflt = {grouped ? 8 : 16, 2};
    Iq3Shape sh = dflt;
    if (env_w) sh.waves = env_w;
    if (env_r) sh.ring = env_r;
    if (waves) sh.waves = waves;
    if (iq3_stream_slots(sh, false) == 0) {
        sh.ring = dflt.ring;
        if (iq3_stream_slots(sh, false) == 0) sh = dflt;
    }
    return sh;
}

// Split-sum workspace, one per (device, stream): partial sums [splits][batch]
// [tiles*64] fp32 followed by one counter per tile (choose_plan keeps every
// plan inside these sizes).
struct Workspace {
    float *partial = nullptr;
    uint32_t *counters = nullptr;
    ShortState sh = {nullptr, nullptr};
};

size_t workspace_partial_floats() { return kWsPartialFloats; }
size_t workspace_counters() { return kWsCounters; }

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// The workspace of (current device, stream), created on first use. Creation
// allocates and clears device memory synchronously, which a stream under graph
// capture cannot do: such a call gets QWG_ERR_CAPTURE and nothing is
// allocated (qwg_workspace_reserve prepares a stream before capture).
int get_workspace(hipStream_t stream, Workspace *out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QWG_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mu);
    auto key = std::make_pair(dev, stream);
    auto it = g_ws.find(key);
    if (it != g_ws.end()) {
        *out = it->second;
        return QWG_OK;
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return QWG_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return QWG_ERR_CAPTURE;
    const size_t pbytes = workspace_partial_floats() * sizeof(float);
    const size_t wbytes = kShortWords * sizeof(uint64_t);
    const size_t cbytes = workspace_counters() * sizeof(uint32_t);
    const size_t ebytes = kShortEpochs * sizeof(uint32_t);
    void *mem = nullptr;
    if (hipMalloc(&mem, pbytes + wbytes + cbytes + ebytes) != hipSuccess) return QWG_ERR_HIP;
    // Counters start at zero and every launch leaves them at zero again; the
    // short calls' tagged words and epochs start at zero (no word carries a
    // tag a call waits for).
    if (hipMemset((uint8_t *)mem + pbytes, 0, wbytes + cbytes + ebytes) != hipSuccess) {
        (void)hipFree(mem);
        return QWG_ERR_HIP;
    }
    Workspace ws;
    ws.partial = (float *)mem;
    ws.sh.words = (uint64_t *)((uint8_t *)mem + pbytes);
    ws.counters = (uint32_t *)((uint8_t *)mem + pbytes + wbytes);
    ws.sh.epochs = (uint32_t *)((uint8_t *)mem + pbytes + wbytes + cbytes);
    g_ws.emplace(key, ws);
    *out = ws;
    return QWG_OK;
}

void fill_shape(GemvArgs &a, const void *w, const float *x, const float *grid, float *y,
                int64_t n_in, int64_t n_out, int block_bytes) {
    a.w = (const uint8_t *)w;
    a.x = x;
    a.grid = grid;
    a.y = y;
    a.n_in = (int)n_in;
    a.n_out = (int)n_out;
    a.nb = (int)(n_in / kQK);
    a.row_bytes = (int64_t)a.nb * block_bytes;
    a.tiles = (int)((n_out + kTileRows - 1) / kTileRows);
    a.splits = 1;
    a.wg_begin = 0;
    a.partial = nullptr;
    a.counters = nullptr;
    a.layout = kLayoutRows;
}

// Splits of an IQ3 GEMV: enough work items (tiles x splits) to give every
// resident workgroup of the stream engine one, at most one split per
// super-block, and partial sums inside the workspace.
int iq3_splits(int tiles, int nb, int slots) {
    if (tiles >= slots) return 1;
    int s = slots / tiles;
    if (s > nb) s = nb;
    if (s < 1) s = 1;
    while (s > 1 && ((size_t)s * tiles * kTileRows > kWsPartialFloats || (size_t)tiles > kWsCounters))
        --s;
    return s;
}

// Splits of a stream-engine problem that would leave workgroup slots idle:
// `factor` items per tile at most (the slots over the launch's tiles), and no
// more than one pipeline stage (`bps` super-blocks) per item, since an item's
// stages run one after another while separate items run side by side.
// Measured on MI355X: a dependent launch of 2048 x 5632 (32 tiles of 22
// super-blocks) took 16 us streaming whole rows.
int stream_splits(int nb, int bps, int64_t factor) {
    static const int env_max = env_int("QWG_STREAM_SPLIT_MAX", 0);  // tuning experiments
    int s = (nb + bps - 1) / bps;
    if ((int64_t)s > factor) s = (int)factor;
    if (env_max && s > env_max) s = env_max;
    return s < 1 ? 1 : s;
}

// Splits and engine shape of a single IQ3_S / IQ4_XS GEMV on the tile layout
// (tiled) or on row-major blocks: none when the tiles alone give every
// resident workgroup of the engine two items; otherwise the split shape and
// as many splits as stream_splits allows within the workspace. Splits 0 when
// the engine's residency is unknown.
struct CbPlan {
    int splits, shape;
};

CbPlan cb_plan(int fmt, bool tiled, int nb, int tiles) {
    CbPlan p = {1, cb_stream_shape(fmt, false)};
    const int slots = cb_stream_slots(fmt, tiled, p.shape);
    if (slots <= 0) return {0, p.shape};
    if (slots <= 2 * tiles) return p;
    p.shape = cb_stream_shape(fmt, true);
    const int ss = cb_stream_slots(fmt, tiled, p.shape);
    if (ss <= 0) return {0, p.shape};
    int sp = stream_splits(nb, p.shape / 40, ss / tiles);
    while (sp > 1 && ((size_t)sp * tiles * kTileRows > kWsPartialFloats || (size_t)tiles > kWsCounters))
        --sp;
    p.splits = sp;
    return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QWG_OK : QWG_ERR_HIP; }

}  // namespace

extern "C" {

int qwg_version(void) { return 100; }

const char *qwg_strerror(int status) {
    switch (status) {
        case QWG_OK: return "ok";
        case QWG_ERR_NULL: return "a required pointer is NULL";
        case QWG_ERR_SHAPE: return "invalid size (n_in must be a multiple of 256 in [256, 65536]; n, n_out >= 1)";
        case QWG_ERR_ALIGN: return "a pointer is not aligned as the call requires";
        case QWG_ERR_BATCH: return "batch must be in 1..8";
        case QWG_ERR_HIP: return "HIP runtime error";
        case QWG_ERR_FORMAT: return "unknown format id";
        case QWG_ERR_GRID:
            return "a codebook value is not exactly representable in fp16 (the GEMV keeps the "
                   "codebook in fp16)";
        case QWG_ERR_TIMEOUT:
            return "a wait of the layer-chain launch gave up (its flags have been reset)";
        case QWG_ERR_CAPTURE:
            return "the stream is being captured and has no split-sum workspace yet "
                   "(qwg_workspace_reserve it before capture, or call qwg_gemm_q4k_noalloc)";
        default: return "unknown status";
    }
}

namespace {

static_assert(QWG_FMT_IQ3_S == kFmtIq3s && QWG_FMT_IQ4_XS == kFmtIq4xs, "format ids");

bool known_format(int fmt) {
    return fmt == QWG_FMT_Q4K || fmt == QWG_FMT_IQ3 || fmt == QWG_FMT_IQ3_XXS ||
           fmt == QWG_FMT_IQ3_S || fmt == QWG_FMT_IQ4_XS;
}

int block_bytes_of(int fmt) {
    switch (fmt) {
        case QWG_FMT_Q4K: return kQ4kBytes;
        case QWG_FMT_IQ3_S: return kIq3sBytes;
        case QWG_FMT_IQ4_XS: return kIq4xsBytes;
        default: return kIq3Bytes;
    }
}

bool codebook_format(int fmt) { return fmt == QWG_FMT_IQ3_S || fmt == QWG_FMT_IQ4_XS; }

}  // namespace

int64_t qwg_row_bytes(int fmt, int64_t n_in) {
    if (!known_format(fmt)) return -QWG_ERR_FORMAT;
    if (n_in <= 0 || n_in % kQK) return -QWG_ERR_SHAPE;
    return (n_in / kQK) * block_bytes_of(fmt);
}

int qwg_plan_splits(int fmt, int64_t n_in, int64_t n_out) {
    if (!known_format(fmt)) return -QWG_ERR_FORMAT;
    int rc = check_gemv_shape(n_in, n_out);
    if (rc) return -rc;
    const int tiles = (int)((n_out + kTileRows - 1) / kTileRows);
    if (codebook_format(fmt)) {
        if (rows_engine_cb(tiles, (int)(n_in / kQK))) return 1;
        const int sp = cb_plan(fmt, false, (int)(n_in / kQK), tiles).splits;
        return sp > 0 ? sp : -QWG_ERR_HIP;
    }
    if (fmt != QWG_FMT_Q4K) {
        if (rows_engine_iq3(tiles, (int)(n_in / kQK))) return 1;
        const int ss = short_splits(tiles, (int)(n_in / kQK));
        if (ss > 0) return ss;
        const int slots = iq3_stream_slots(iq3_shape(false, 0), false);
        if (slots <= 0) return -QWG_ERR_HIP;
        return iq3_splits(tiles, (int)(n_in / kQK), slots);
    }
    if (rows_engine(tiles, (int)(n_in / kQK))) return 1;
    const int ss = short_splits(tiles, (int)(n_in / kQK));
    return ss > 0 ? ss : choose_splits(tiles, (int)(n_in / kQK));
}

int qwg_workspace_reserve(void *stream) {
    Workspace ws;
    return get_workspace((hipStream_t)stream, &ws);
}

int qwg_workspace_release(void *stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QWG_ERR_HIP;
    void *mem = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_ws_mu);
        auto it = g_ws.find(std::make_pair(dev, (hipStream_t)stream));
        if (it == g_ws.end()) return QWG_OK;
        mem = it->second.partial;
        g_ws.erase(it);
    }
    // hipFree waits for the device to finish the work that may still use it
    return hip_status(hipFree(mem));
}

int qwg_dequant_q4k(const void *src, float *dst, int64_t n, void *stream) {
    if (!src || !dst) return QWG_ERR_NULL;
    if (n <= 0 || n % kQK) return QWG_ERR_SHAPE;
    if (!aligned(src, 16) || !aligned(dst, 16)) return QWG_ERR_ALIGN;
    return hip_status(launch_q4k_dequant((const uint8_t *)src, dst, n / kQK, (hipStream_t)stream));
}

namespace {

int iq3_dequant(const void *src, const float *grid, float *dst, int64_t n, bool xxs,
                void *stream) {
    if (!src || !grid || !dst) return QWG_ERR_NULL;
    if (n <= 0 || n % kQK) return QWG_ERR_SHAPE;
    if (!aligned(src, 2) || !aligned(grid, 16) || !aligned(dst, 16)) return QWG_ERR_ALIGN;
    return hip_status(
        launch_iq3_dequant((const uint8_t *)src, grid, dst, n / kQK, xxs, (hipStream_t)stream));
}

}  // namespace

int qwg_dequant_iq3(const void *src, const float *grid, float *dst, int64_t n, void *stream) {
    return iq3_dequant(src, grid, dst, n, false, stream);
}

int qwg_dequant_iq3_xxs(const void *src, const float *grid, float *dst, int64_t n, void *stream) {
    return iq3_dequant(src, grid, dst, n, true, stream);
}

}  // extern "C"

namespace {

// Split-sum scratch of qwg_gemm_q4k_noalloc: partial sums (kScratchFloats),
// the short calls' tagged words (kShortWords x 8 bytes), tile counters
// (kScratchCounters) and the short calls' tile epochs (kShortEpochs), one copy
// per GPU in the library's code object. Host code never uses the array's name
// as an address: each device's address comes from hipGetSymbolAddress
// (scratch_of). Everything after the partial sums starts at zero (cleared when a
// device is first used); every launch leaves the counters at zero. The largest split plan of qwg_gemm_q4k needs fewer than 2,304 x 64
// partial sums (batch 1) and fewer than 256 tiles, so these sizes cover every
// shape; a plan that did not fit would be rejected (QWG_ERR_SHAPE).
constexpr size_t kScratchFloats = (size_t)4096 * kTileRows;
constexpr size_t kScratchCounters = 4096;
constexpr size_t kScratchZeroed = 2 * kShortWords + kScratchCounters + kShortEpochs;
static __device__ __align__(256) uint32_t scratch[kScratchFloats + kScratchZeroed];

__global__ void zero_u32_kernel(uint32_t *p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

std::mutex g_scratch_mu;
std::map<int, uint32_t *> g_scratch;

// This device's copy of `scratch` (set up on the first call on the device:
// symbol address, then a fill kernel that zeroes the counters, enqueued on the
// caller's stream ahead of the call's own kernels).
int scratch_of(hipStream_t stream, Workspace *out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QWG_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch.find(dev);
    uint32_t *base = nullptr;
    if (it != g_scratch.end()) {
        base = it->second;
    } else {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return QWG_ERR_HIP;
        base = (uint32_t *)ptr;
        hipLaunchKernelGGL(zero_u32_kernel, dim3(64), dim3(256), 0, stream,
                           base + kScratchFloats, (int)kScratchZeroed);
        if (hipGetLastError() != hipSuccess) return QWG_ERR_HIP;
        g_scratch.emplace(dev, base);
    }
    out->partial = (float *)base;
    out->sh.words = (uint64_t *)(base + kScratchFloats);
    out->counters = base + kScratchFloats + 2 * kShortWords;
    out->sh.epochs = out->counters + kScratchCounters;
    return QWG_OK;
}

// qwg_gemm_q4k, its split sums in the stream's workspace (noalloc = false) or
// in the static scratch (noalloc = true).
int gemm_q4k(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out, int batch,
             hipStream_t stream, bool noalloc) {
    if (!y || !x || !w) return QWG_ERR_NULL;
    int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (batch < 1 || batch > QWG_MAX_BATCH) return QWG_ERR_BATCH;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return QWG_ERR_ALIGN;
    GemvArgs a;
    fill_shape(a, w, x, nullptr, y, n_in, n_out, kQ4kBytes);
    // Engine: the vector ALUs for batch 1, and for batch 2 on a matrix of many
    // tiles (8 wavefronts per tile; measured on the LM head, 500 tiles, cold
    // weights: 12.4 us against 14.2-15.8 us on the matrix cores, while on the
    // layer shapes of 32-88 tiles and at batch 3..8 the matrix cores win or
    // tie: bench.py --workload gemm_ab); otherwise the matrix cores.
    if (batch == 1 && rows_engine(a.tiles, a.nb)) return hip_status(launch_q4k_rows(a, false, stream));
    if (batch == 1) {
        const int ss = short_splits(a.tiles, a.nb);
        if (ss > 0) {
            a.splits = ss;
            Workspace ws;
            if (ss > 1) {
                rc = noalloc ? scratch_of(stream, &ws) : get_workspace(stream, &ws);
                if (rc) return rc;
            }
            return hip_status(launch_q4k_short(a, ws.sh, false, stream));
        }
    }
    const bool valu = batch == 1 || (batch == 2 && a.tiles >= kValuBatch2Tiles);
    const bool mstream = !valu && !mfma_tile_engine();
    const int ring = mstream_ring();
    int waves = kQ4kWavesSmall;
    if (valu) {
        const Plan plan = choose_plan(a.tiles, a.nb, batch);
        a.splits = plan.splits;
        waves = batch == 1 ? plan.waves : 8;
    } else if (mstream) {
        const int slots = q4k_mstream_slots(ring);
        if (slots <= 0) return QWG_ERR_HIP;
        a.splits = mstream_splits(a.tiles, a.nb, batch, slots);
    } else {
        a.splits = mfma_splits(a.tiles, a.nb, batch);
    }
    if (a.splits > 1) {
        Workspace ws;
        if (noalloc) {
            if ((size_t)a.splits * batch * a.tiles * kTileRows > kScratchFloats ||
                (size_t)a.tiles > kScratchCounters)
                return QWG_ERR_SHAPE;
            rc = scratch_of(stream, &ws);
        } else {
            rc = get_workspace(stream, &ws);
        }
        if (rc) return rc;
        a.partial = ws.partial;
        a.counters = ws.counters;
    }
    if (mstream) {
        const GroupArgs none = {nullptr, nullptr, nullptr};
        return hip_status(launch_q4k_mstream(none, a, a.tiles * a.splits, batch, ring, a.splits > 1,
                                             stream));
    }
    if (!valu) return hip_status(launch_mfma(a, batch, stream));
    if (batch == 1 && a.splits == 1 && use_stream_engine()) {
        const StreamShape sh = stream_shape(false);
        const GroupArgs none = {nullptr, nullptr, nullptr};
        return hip_status(launch_q4k_stream(none, a, a.tiles, sh.waves, sh.ring, false, stream));
    }
    return hip_status(launch_q4k_gemv(a, batch, waves, stream));
}

}  // namespace

extern "C" {

int qwg_gemm_q4k(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out, int batch,
                 void *stream) {
    return gemm_q4k(y, x, w, n_in, n_out, batch, (hipStream_t)stream, false);
}

int qwg_gemm_q4k_noalloc(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                         int batch, void *stream) {
    return gemm_q4k(y, x, w, n_in, n_out, batch, (hipStream_t)stream, true);
}

int qwg_gemm_q4k_ex(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                    int batch, int waves, int splits, void *stream) {
    if (!y || !x || !w) return QWG_ERR_NULL;
    int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (batch < 1 || batch > QWG_MAX_BATCH) return QWG_ERR_BATCH;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return QWG_ERR_ALIGN;
    GemvArgs a;
    fill_shape(a, w, x, nullptr, y, n_in, n_out, kQ4kBytes);
    const int ring = mstream_ring();
    const bool mstream = waves == kWavesMstream || (waves == 0 && batch >= 2 && !mfma_tile_engine());
    const bool mfma = !mstream && (waves == kWavesMfma || waves == kWavesMfma2 ||
                                   (waves == 0 && batch >= 2));
    if ((mfma || mstream) && batch < 2) return QWG_ERR_SHAPE;
    const Plan autoplan = choose_plan(a.tiles, a.nb, batch);
    if (splits == 0) {
        if (mstream) {
            const int slots = q4k_mstream_slots(ring);
            if (slots <= 0) return QWG_ERR_HIP;
            splits = mstream_splits(a.tiles, a.nb, batch, slots);
        } else {
            splits = mfma ? mfma_splits(a.tiles, a.nb, batch) : autoplan.splits;
        }
    }
    if (waves == 0 && !mfma) waves = autoplan.waves;
    if (!mfma && !mstream && waves != 4 && waves != 8 && waves != 16) return QWG_ERR_SHAPE;
    if (splits < 1 || splits > a.nb) return QWG_ERR_SHAPE;
    if (splits > 1 && ((size_t)splits * batch * a.tiles * kTileRows > kWsPartialFloats ||
                       (size_t)a.tiles > kWsCounters))
        return QWG_ERR_SHAPE;
    a.splits = splits;
    if (splits > 1) {
        Workspace ws;
        rc = get_workspace((hipStream_t)stream, &ws);
        if (rc) return rc;
        a.partial = ws.partial;
        a.counters = ws.counters;
    }
    if (mstream) {
        const GroupArgs none = {nullptr, nullptr, nullptr};
        return hip_status(launch_q4k_mstream(none, a, a.tiles * a.splits, batch, ring, a.splits > 1,
                                             (hipStream_t)stream));
    }
    if (mfma) return hip_status(launch_mfma(a, batch, (hipStream_t)stream, waves));
    return hip_status(launch_q4k_gemv(a, batch, waves, (hipStream_t)stream));
}

int qwg_gemv_q4k(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                 void *stream) {
    return qwg_gemm_q4k(y, x, w, n_in, n_out, 1, stream);
}

int64_t qwg_tiled_bytes(int fmt, int64_t n_in, int64_t n_out) {
    if (!known_format(fmt)) return -QWG_ERR_FORMAT;
    const int rc = check_gemv_shape(n_in, n_out);
    if (rc) return -rc;
    const int tb = (fmt == QWG_FMT_IQ3 || fmt == QWG_FMT_IQ3_XXS) ? kIq3TileBlock : block_bytes_of(fmt);
    return ((n_out + kTileRows - 1) / kTileRows) * kTileRows * (n_in / kQK) * tb;
}

int qwg_pack_q4k_tiles(void *dst, const void *src, int64_t n_in, int64_t n_out, void *stream) {
    if (!dst || !src) return QWG_ERR_NULL;
    const int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (!aligned(dst, 16) || !aligned(src, 16)) return QWG_ERR_ALIGN;
    return hip_status(launch_q4k_pack_tiles((const uint8_t *)src, (uint8_t *)dst, (int)(n_in / kQK),
                                            (int)n_out, (hipStream_t)stream));
}

int qwg_gemm_q4k_tiled(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                       int batch, void *stream) {
    if (!y || !x || !w) return QWG_ERR_NULL;
    const int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (batch < 1 || batch > QWG_MAX_BATCH) return QWG_ERR_BATCH;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return QWG_ERR_ALIGN;
    if (batch == 1) return qwg_gemv_q4k_tiled(y, x, w, n_in, n_out, stream);
    GemvArgs a;
    fill_shape(a, w, x, nullptr, y, n_in, n_out, kQ4kBytes);
    a.layout = kLayoutTiles;
    const bool mstream = !mfma_tile_engine();
    const int ring = mstream_ring();
    if (mstream) {
        const int slots = q4k_mstream_slots(ring);
        if (slots <= 0) return QWG_ERR_HIP;
        a.splits = mstream_splits(a.tiles, a.nb, batch, slots);
    } else {
        a.splits = mfma_splits(a.tiles, a.nb, batch);
    }
    if (a.splits > 1) {
        Workspace ws;
        const int wrc = get_workspace((hipStream_t)stream, &ws);
        if (wrc) return wrc;
        a.partial = ws.partial;
        a.counters = ws.counters;
    }
    if (mstream) {
        const GroupArgs none = {nullptr, nullptr, nullptr};
        return hip_status(launch_q4k_mstream(none, a, a.tiles * a.splits, batch, ring, a.splits > 1,
                                             (hipStream_t)stream));
    }
    return hip_status(launch_mfma(a, batch, (hipStream_t)stream, 0, true));
}

int qwg_gemv_q4k_tiled(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                       void *stream) {
    if (!y || !x || !w) return QWG_ERR_NULL;
    const int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return QWG_ERR_ALIGN;
    GemvArgs a;
    fill_shape(a, w, x, nullptr, y, n_in, n_out, kQ4kBytes);
    a.layout = kLayoutTiles;
    if (rows_engine(a.tiles, a.nb)) return hip_status(launch_q4k_rows(a, true, (hipStream_t)stream));
    const int ss = short_splits(a.tiles, a.nb);
    if (ss > 0) {
        a.splits = ss;
        Workspace ws;
        if (ss > 1) {
            const int wrc = get_workspace((hipStream_t)stream, &ws);
            if (wrc) return wrc;
        }
        return hip_status(launch_q4k_short(a, ws.sh, true, (hipStream_t)stream));
    }
    const StreamShape sh = stream_shape(false);
    int cus = 0;
    const int64_t slots = (int64_t)q4k_stream_residency(sh.waves, sh.ring, &cus) * cus;
    if (slots > 2 * (int64_t)a.tiles) {
        int sp = stream_splits(a.nb, sh.waves / 4, slots / a.tiles);
        while (sp > 1 && ((size_t)sp * a.tiles * kTileRows > kWsPartialFloats ||
                          (size_t)a.tiles > kWsCounters))
            --sp;
        a.splits = sp;
    }
    if (a.splits > 1) {
        Workspace ws;
        const int wrc = get_workspace((hipStream_t)stream, &ws);
        if (wrc) return wrc;
        a.partial = ws.partial;
        a.counters = ws.counters;
    }
    const GroupArgs none = {nullptr, nullptr, nullptr};
    return hip_status(launch_q4k_stream(none, a, a.tiles * a.splits, sh.waves, sh.ring,
                                        a.splits > 1, (hipStream_t)stream));
}

namespace {

int iq3_gemv(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
             int64_t n_out, int waves, int splits, int layout, void *stream) {
    const bool tiled = layout == kLayoutTiles;
    if (!y || !x || !w || !grid) return QWG_ERR_NULL;
    int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (!aligned(w, tiled ? 16 : 2) || !aligned(x, 16) || !aligned(grid, 16) || !aligned(y, 4))
        return QWG_ERR_ALIGN;
    if (waves != 0 && waves != 4 && waves != 8 && waves != 16) return QWG_ERR_SHAPE;
    GemvArgs a;
    fill_shape(a, w, x, grid, y, n_in, n_out, kIq3Bytes);
    if (splits < 0 || splits > a.nb) return QWG_ERR_SHAPE;
    if (splits > 1 && ((size_t)splits * a.tiles * kTileRows > kWsPartialFloats ||
                       (size_t)a.tiles > kWsCounters))
        return QWG_ERR_SHAPE;
    a.layout = layout;
    if (waves == 0 && splits == 0) {
        // automatic plan: the short-call kernels when the matrix fits them
        if (rows_engine_iq3(a.tiles, a.nb)) return hip_status(launch_iq3_rows(a, grid, (hipStream_t)stream));
        const int ss = short_splits(a.tiles, a.nb);
        if (ss > 0) {
            a.splits = ss;
            Workspace ws;
            if (ss > 1) {
                rc = get_workspace((hipStream_t)stream, &ws);
                if (rc) return rc;
            }
            return hip_status(launch_iq3_short(a, ws.sh, grid, (hipStream_t)stream));
        }
    }
    const Iq3Shape sh = iq3_shape(false, waves);
    const int slots = iq3_stream_slots(sh, tiled);
    if (slots <= 0) return QWG_ERR_HIP;
    if (splits == 0) splits = iq3_splits(a.tiles, a.nb, slots);
    a.splits = splits;
    if (splits > 1) {
        Workspace ws;
        rc = get_workspace((hipStream_t)stream, &ws);
        if (rc) return rc;
        a.partial = ws.partial;
        a.counters = ws.counters;
    }
    const GroupArgs none = {nullptr, nullptr, nullptr};
    return hip_status(
        launch_iq3_stream(none, a, grid, a.tiles * splits, sh, tiled, (hipStream_t)stream));
}

}  // namespace

int qwg_gemv_iq3_ex(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                    int64_t n_out, int waves, int splits, void *stream) {
    return iq3_gemv(y, x, w, grid, n_in, n_out, waves, splits, kLayoutRows, stream);
}

int qwg_gemv_iq3(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                 int64_t n_out, void *stream) {
    return iq3_gemv(y, x, w, grid, n_in, n_out, 0, 0, kLayoutRows, stream);
}

int qwg_gemv_iq3_xxs(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                     int64_t n_out, void *stream) {
    return iq3_gemv(y, x, w, grid, n_in, n_out, 0, 0, kLayoutRowsXxs, stream);
}

int qwg_gemv_iq3_tiled(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                       int64_t n_out, void *stream) {
    return iq3_gemv(y, x, w, grid, n_in, n_out, 0, 0, kLayoutTiles, stream);
}

namespace {

int iq3_pack(void *dst, const void *src, int64_t n_in, int64_t n_out, bool xxs, void *stream) {
    if (!dst || !src) return QWG_ERR_NULL;
    const int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (!aligned(dst, 16) || !aligned(src, 2)) return QWG_ERR_ALIGN;
    return hip_status(launch_iq3_pack_tiles((const uint8_t *)src, (uint8_t *)dst, (int)(n_in / kQK),
                                            (int)n_out, xxs, (hipStream_t)stream));
}

}  // namespace

int qwg_pack_iq3_tiles(void *dst, const void *src, int64_t n_in, int64_t n_out, void *stream) {
    return iq3_pack(dst, src, n_in, n_out, false, stream);
}

int qwg_pack_iq3_xxs_tiles(void *dst, const void *src, int64_t n_in, int64_t n_out, void *stream) {
    return iq3_pack(dst, src, n_in, n_out, true, stream);
}

int qwg_encode_iq3(void *dst, const float *x, const float *grid, int64_t n_rows, int64_t n_in,
                   void *stream) {
    if (!dst || !x || !grid) return QWG_ERR_NULL;
    if (n_rows < 1 || n_rows > QWG_MAX_N_OUT || n_in <= 0 || n_in % kQK || n_in > QWG_MAX_N_IN)
        return QWG_ERR_SHAPE;
    if (!aligned(x, 4) || !aligned(grid, 16)) return QWG_ERR_ALIGN;
    return hip_status(launch_iq3_encode(x, grid, (uint8_t *)dst, n_rows * (n_in / kQK),
                                        (hipStream_t)stream));
}

// ------------------------------------------------------------------ IQ3_S, IQ4_XS

namespace {

int cb_dequant(int fmt, const void *src, const float *tab, float *dst, int64_t n, void *stream) {
    if (!src || !tab || !dst) return QWG_ERR_NULL;
    if (n <= 0 || n % kQK) return QWG_ERR_SHAPE;
    if (!aligned(src, fmt == QWG_FMT_IQ4_XS ? 4 : 2) || !aligned(tab, 16) || !aligned(dst, 16))
        return QWG_ERR_ALIGN;
    const hipError_t e =
        fmt == QWG_FMT_IQ3_S
            ? launch_iq3s_dequant((const uint8_t *)src, tab, dst, n / kQK, (hipStream_t)stream)
            : launch_iq4xs_dequant((const uint8_t *)src, tab, dst, n / kQK, (hipStream_t)stream);
    return hip_status(e);
}

int cb_pack(int fmt, void *dst, const void *src, int64_t n_in, int64_t n_out, void *stream) {
    if (!dst || !src) return QWG_ERR_NULL;
    const int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (!aligned(dst, 16) || !aligned(src, 2)) return QWG_ERR_ALIGN;
    return hip_status(launch_cb_pack_tiles(fmt, (const uint8_t *)src, (uint8_t *)dst,
                                           (int)(n_in / kQK), (int)n_out, (hipStream_t)stream));
}

int cb_gemv(int fmt, bool tiled, float *y, const float *x, const void *w, const float *tab,
            int64_t n_in, int64_t n_out, void *stream) {
    if (!y || !x || !w || !tab) return QWG_ERR_NULL;
    int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(tab, 16) || !aligned(y, 4))
        return QWG_ERR_ALIGN;
    GemvArgs a;
    fill_shape(a, w, x, tab, y, n_in, n_out, block_bytes_of(fmt));
    a.layout = tiled ? kLayoutTiles : kLayoutRows;
    if (rows_engine_cb(a.tiles, a.nb)) return hip_status(launch_cb_rows(fmt, a, tab, (hipStream_t)stream));
    const CbPlan plan = cb_plan(fmt, tiled, a.nb, a.tiles);
    if (plan.splits <= 0) return QWG_ERR_HIP;
    a.splits = plan.splits;
    if (a.splits > 1) {
        Workspace ws;
        rc = get_workspace((hipStream_t)stream, &ws);
        if (rc) return rc;
        a.partial = ws.partial;
        a.counters = ws.counters;
    }
    const GroupArgs none = {nullptr, nullptr, nullptr};
    return hip_status(
        launch_cb_stream(fmt, tiled, plan.shape, none, a, tab, a.tiles * a.splits,
                         (hipStream_t)stream));
}

}  // namespace

int qwg_dequant_iq3s(const void *src, const float *grid, float *dst, int64_t n, void *stream) {
    return cb_dequant(QWG_FMT_IQ3_S, src, grid, dst, n, stream);
}

int qwg_dequant_iq4xs(const void *src, const float *table, float *dst, int64_t n, void *stream) {
    return cb_dequant(QWG_FMT_IQ4_XS, src, table, dst, n, stream);
}

int qwg_pack_iq3s_tiles(void *dst, const void *src, int64_t n_in, int64_t n_out, void *stream) {
    return cb_pack(QWG_FMT_IQ3_S, dst, src, n_in, n_out, stream);
}

int qwg_pack_iq4xs_tiles(void *dst, const void *src, int64_t n_in, int64_t n_out, void *stream) {
    return cb_pack(QWG_FMT_IQ4_XS, dst, src, n_in, n_out, stream);
}

int qwg_gemv_iq3s(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                  int64_t n_out, void *stream) {
    return cb_gemv(QWG_FMT_IQ3_S, false, y, x, w, grid, n_in, n_out, stream);
}

int qwg_gemv_iq4xs(float *y, const float *x, const void *w, const float *table, int64_t n_in,
                   int64_t n_out, void *stream) {
    return cb_gemv(QWG_FMT_IQ4_XS, false, y, x, w, table, n_in, n_out, stream);
}

int qwg_gemv_iq3s_tiled(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                        int64_t n_out, void *stream) {
    return cb_gemv(QWG_FMT_IQ3_S, true, y, x, w, grid, n_in, n_out, stream);
}

int qwg_gemv_iq4xs_tiled(float *y, const float *x, const void *w, const float *table,
                         int64_t n_in, int64_t n_out, void *stream) {
    return cb_gemv(QWG_FMT_IQ4_XS, true, y, x, w, table, n_in, n_out, stream);
}

// ------------------------------------------------------------------ grouped GEMV

struct qwg_group {
    int device;
    int fmt;              // QWG_FMT_Q4K, QWG_FMT_IQ3, QWG_FMT_IQ3_S or QWG_FMT_IQ4_XS
    int layout;           // kLayoutRows or kLayoutTiles
    const float *grid;    // IQ3 / IQ3_S: the grid, IQ4_XS: the table every member uses
    void *dev_mem;        // GemvArgs[count], uint32_t map[positions] (and tile[positions]),
                          // then the split members' partial sums and tile counters
    GroupArgs args;
    int count;
    int workgroups;       // 64-row tiles of one run
    int positions;        // work-list length of a launch (items, plus holes of a schedule)
    int max_nb;
    bool split;           // some member splits its rows' sums
    int waves, ring;      // Q4_K stream engine shape of the launch
    int cb_shape;         // IQ3_S / IQ4_XS engine shape of the launch (10 * waves + ring)
    int mring;            // batched: ring stages of the persistent stream (0: per-tile pipeline)
    int batch;            // activation rows per member (2..8: the matrix-core engine)
    int cols;             // its super-block columns per stage
};

namespace {

// Static schedule of a grouped Q4_K stream launch. Resident workgroup b walks
// positions b, b + G, b + 2G, ... (G = resident workgroups of the launch).
// Measured on MI355X, workgroups that share a CU do not progress at the same
// rate: wavefronts issue oldest first, so the workgroup dispatched first to a
// CU streams its tiles about three times as fast as the seventh, and equal
// shares leave the young ones running alone at the end with too few bytes in
// flight. Workgroup b is the (b / CUs)-th to arrive on its CU, so its share is
// weighted by a ramp from 1 + skew (first) to 1 - skew (last); tiles, longest
// rows first, go one by one to the workgroup furthest below its weighted share.
// Positions past the end of a workgroup's list hold kNoItem. Measured on the
// 155-GEMV TinyLlama stream: skew 0 (plain longest-first balance) 106.4 us,
// 0.3 104.3, 0.5 102.3, 0.7 101.7, 0.85 101.9; equal round-robin shares 104.8.
// Re-measured with the tile layout (same box, two rounds): 0.5 88.6 / 88.6 us,
// 0.6 88.5 / 88.1, 0.7 89.0 / 89.0, 0.8 89.0 / 89.0. A per-wavefront cycle
// count still shows the youngest workgroup of each CU (one item) finishing
// ~25% before the others. QWG_STREAM_SKEW overrides it (tuning experiments).
constexpr double kAgeSkew = 0.6;

double skew_env(const char *name, double dflt) {
    const char *e = getenv(name);
    const double d = e ? atof(e) : dflt;
    return d < 0.0 ? 0.0 : (d > 0.95 ? 0.95 : d);
}

void stream_schedule(const std::vector<GemvArgs> &probs, const std::vector<int> &order,
                     int64_t total, int per_cu, int cus, double skew_arg,
                     std::vector<uint32_t> &map, std::vector<uint32_t> &tile) {
    const int64_t grid = (int64_t)per_cu * cus;
    if (grid < 1 || total <= grid) {
        // one item (or none) per workgroup: the sorted list itself
        map.resize((size_t)total);
        tile.resize((size_t)total);
        size_t k = 0;
        for (int i : order)
            for (int t = 0; t < probs[i].tiles * probs[i].splits; ++t, ++k) {
                map[k] = (uint32_t)i;
                tile[k] = (uint32_t)t;
            }
        return;
    }
    const double skew = per_cu > 1 ? skew_arg : 0.0;
    std::vector<double> target((size_t)grid);
    double wsum = 0.0;
    for (int64_t b = 0; b < grid; ++b) {
        const int rank = (int)(b / cus);
        target[b] = 1.0 + skew * (double)(per_cu - 1 - 2 * rank) / (double)(per_cu - 1 > 0 ? per_cu - 1 : 1);
        wsum += target[b];
    }
    double work = 0.0;
    for (int i : order) work += (double)probs[i].tiles * probs[i].nb;
    auto item_blocks = [&](int i) {
        return (double)((probs[i].nb + probs[i].splits - 1) / probs[i].splits);
    };
    for (double &t : target) t *= work / wsum;
    std::priority_queue<std::pair<double, int64_t>> deficit;
    for (int64_t b = 0; b < grid; ++b) deficit.push({target[b], -b});
    std::vector<double> load((size_t)grid, 0.0);
    std::vector<std::vector<std::pair<uint32_t, uint32_t>>> lists((size_t)grid);
    size_t longest = 0;
    for (int i : order)
        for (int t = 0; t < probs[i].tiles * probs[i].splits; ++t) {
            const int64_t b = -deficit.top().second;
            deficit.pop();
            lists[b].push_back({(uint32_t)i, (uint32_t)t});
            load[b] += item_blocks(i);
            deficit.push({target[b] - load[b], -b});
            longest = std::max(longest, lists[b].size());
        }
    map.assign((size_t)grid * longest, kNoItem);
    tile.assign((size_t)grid * longest, 0u);
    for (int64_t b = 0; b < grid; ++b)
        for (size_t j = 0; j < lists[b].size(); ++j) {
            map[j * grid + b] = lists[b][j].first;
            tile[j * grid + b] = lists[b][j].second;
        }
}

// True if v converts to binary16 and back unchanged: zero; a normal fp16
// magnitude (2^-14 .. 65504) whose significand fits 11 bits; or a subnormal
// fp16 value (a multiple of 2^-24 below 2^-14). Infinities and NaN are
// rejected.
bool fp16_exact_host(float v) {
    if (v == 0.0f) return true;
    float a = v < 0.0f ? -v : v;
    if (!(a <= 65504.0f)) return false;
    if (a < 6.103515625e-05f) {
        const float m = a * 16777216.0f;   // exact (power-of-two scale)
        return m == (float)(int64_t)m;
    }
    uint32_t bits;
    memcpy(&bits, &a, sizeof bits);
    return (bits & 0x1FFFu) == 0;
}

// The codebook of an IQ3 / IQ3_S / IQ4_XS group, copied to the host and
// checked: the GEMV engines hold it in fp16.
int check_codebook(int fmt, const float *grid) {
    const size_t n = fmt == QWG_FMT_IQ3_S ? 512 * 4 : fmt == QWG_FMT_IQ4_XS ? 16 : 256 * 4;
    std::vector<float> h(n);
    if (hipMemcpy(h.data(), grid, n * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
        return QWG_ERR_HIP;
    for (float v : h)
        if (!fp16_exact_host(v)) return QWG_ERR_GRID;
    return QWG_OK;
}

// Work list of a batched group. Workgroup b runs on XCD b % 8 (workgroups are
// dispatched round-robin over the eight XCDs, each with its own L2) and takes
// position b (one workgroup per position) or, on the persistent stream whose
// grid is a multiple of 8, positions b, b + n, ...: always positions
// 8j + b % 8. Each XCD gets a contiguous run of the
// member-major item list holding about an eighth of the weight bytes, so a
// member's activations (up to 8 x 22 KB per member) are fetched into one or
// two L2s rather than all eight; within a run, members keep the longest-rows-
// first order. Shorter runs end in holes (kNoItem).
void xcd_schedule(const std::vector<GemvArgs> &probs, const std::vector<int> &order,
                  std::vector<uint32_t> &map, std::vector<uint32_t> &tile) {
    int64_t total = 0;
    for (int i : order) total += (int64_t)probs[i].tiles * probs[i].nb;
    std::vector<std::vector<std::pair<uint32_t, uint32_t>>> run(8);
    int64_t cum = 0;
    for (int i : order) {
        for (int t = 0; t < probs[i].tiles; ++t) {
            const int64_t mid2 = 2 * cum + probs[i].nb;   // twice the item's cost midpoint
            const int x = (int)std::min<int64_t>(7, mid2 * 8 / (2 * std::max<int64_t>(total, 1)));
            run[(size_t)x].push_back({(uint32_t)i, (uint32_t)t});
            cum += probs[i].nb;
        }
    }
    size_t len = 0;
    for (const auto &r : run) len = std::max(len, r.size());
    map.assign(8 * len, kNoItem);
    tile.assign(8 * len, 0u);
    for (size_t x = 0; x < 8; ++x)
        for (size_t j = 0; j < run[x].size(); ++j) {
            map[8 * j + x] = run[x][j].first;
            tile[8 * j + x] = run[x][j].second;
        }
}

int group_create(int fmt, int layout, const qwg_gemv_desc *descs, int count, const float *grid,
                 qwg_group **out, int batch = 1) {
    const bool cb = codebook_format(fmt);
    const bool iq3 = fmt == QWG_FMT_IQ3 || cb;   // round-robin schedule, grid/table argument
    const int block_bytes = block_bytes_of(fmt);
    // row-major IQ3 blocks need 2-byte alignment; tile layouts and row-major
    // IQ3_S / IQ4_XS (whose engine copies 16-byte granules from the start) 16
    const uintptr_t w_align = iq3 && !cb && layout == kLayoutRows ? 2 : 16;
    std::vector<GemvArgs> probs((size_t)count);
    int64_t total = 0;
    int max_nb = 1;
    for (int i = 0; i < count; ++i) {
        const qwg_gemv_desc &d = descs[i];
        if (!d.y || !d.x || !d.w) return QWG_ERR_NULL;
        int rc = check_gemv_shape(d.n_in, d.n_out);
        if (rc) return rc;
        if (!aligned(d.w, w_align) || !aligned(d.x, 16) || !aligned(d.y, 4)) return QWG_ERR_ALIGN;
        fill_shape(probs[i], d.w, d.x, grid, d.y, d.n_in, d.n_out, block_bytes);
        probs[i].layout = layout;
        total += probs[i].tiles;
        if (probs[i].nb > max_nb) max_nb = probs[i].nb;
    }
    if (total > (int64_t)1 << 30) return QWG_ERR_SHAPE;
    if (iq3) {
        const int rc = check_codebook(fmt, grid);
        if (rc) return rc;
    }
    // Batched members run on the matrix-core engine, one workgroup per tile
    // (a stream has thousands of tiles, so none of them splits).
    const bool batched = batch >= 2;
    const bool stream = !batched && !iq3 && (layout == kLayoutTiles || use_stream_engine());
    // Launches with fewer tiles than resident workgroups split the row sums of
    // their members (at most one pipeline stage per item), as a single GEMV
    // does; a member's partial sums and tile counters live in the group's
    // device memory.
    int64_t slots = 0, bps = 1;
    int per_cu = 0, cus = 0;
    StreamShape ssh = {4, 2};
    int cb_shape = 0;
    if (cb) {
        // as a single GEMV: the split shape when the members' tiles leave
        // resident workgroups idle
        cb_shape = cb_stream_shape(fmt, false);
        slots = cb_stream_slots(fmt, layout == kLayoutTiles, cb_shape);
        if (slots > 2 * total) {
            cb_shape = cb_stream_shape(fmt, true);
            slots = cb_stream_slots(fmt, layout == kLayoutTiles, cb_shape);
        }
        if (slots <= 0) return QWG_ERR_HIP;
        bps = cb_shape / 40;
    } else if (iq3) {
        const Iq3Shape ish = iq3_shape(true, 0);
        slots = iq3_stream_slots(ish, layout == kLayoutTiles);
        bps = ish.waves / 4;
    } else if (stream) {
        ssh = stream_shape(true);
        per_cu = q4k_stream_residency(ssh.waves, ssh.ring, &cus);
        slots = (int64_t)per_cu * cus;
        // A launch that has to split its sums runs 8-wavefront workgroups (two
        // super-blocks per stage): measured on the dependent per-layer
        // launches of the TinyLlama stream, 723 us with 4 wavefronts, 610 us
        // with 8.
        if (slots > 2 * total && !stream_shape_overridden()) {
            ssh = {8, 2};
            per_cu = q4k_stream_residency(ssh.waves, ssh.ring, &cus);
            slots = (int64_t)per_cu * cus;
        }
        bps = ssh.waves / 4;
    }
    size_t partial_floats = 0, counters = 0;
    int64_t items = 0;
    bool split = false;
    for (int i = 0; i < count; ++i) {
        if (!batched && slots > 2 * total)
            probs[i].splits = stream_splits(probs[i].nb, (int)bps, slots / total);
        if (probs[i].splits > 1) {
            split = true;
            partial_floats += (size_t)probs[i].splits * probs[i].tiles * kTileRows;
            counters += (size_t)probs[i].tiles;
        }
        items += (int64_t)probs[i].tiles * probs[i].splits;
    }
    if (items > (int64_t)1 << 30) return QWG_ERR_SHAPE;
    // Work items of the longest rows first, so that short ones fill the tail.
    std::vector<int> order((size_t)count);
    for (int i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return probs[a].nb > probs[b].nb; });
    int64_t wg = 0;
    for (int i : order) {
        probs[i].wg_begin = (int)wg;
        wg += (int64_t)probs[i].tiles * probs[i].splits;
    }
    // IQ3 groups keep the plain longest-first round robin: measured on the IQ3
    // stream (two workgroups per CU) the balanced schedule ran 126 us against
    // 114 us, and any age skew only slowed it further.
    std::vector<uint32_t> map, tile;
    const bool mstream = batched && !mfma_tile_engine();
    static const int env_xcd = env_int("QWG_XCD_MAP", 1);   // 0: plain list (A/B tuning)
    if (batched && env_xcd) {
        xcd_schedule(probs, order, map, tile);
    } else if (stream) {
        static const double skew = skew_env("QWG_STREAM_SKEW", kAgeSkew);
        stream_schedule(probs, order, items, per_cu, cus, skew, map, tile);
    } else {
        map.resize((size_t)items);
        for (int i : order)
            for (int64_t t = 0; t < (int64_t)probs[i].tiles * probs[i].splits; ++t)
                map[(size_t)(probs[i].wg_begin + t)] = (uint32_t)i;
    }
    const int64_t positions = (int64_t)map.size();
    if (positions > (int64_t)1 << 30) return QWG_ERR_SHAPE;
    const size_t pbytes = sizeof(GemvArgs) * (size_t)count;
    const size_t mbytes = sizeof(uint32_t) * (size_t)positions;
    const size_t tbytes = tile.empty() ? 0 : mbytes;
    const size_t wbase = (pbytes + mbytes + tbytes + 255) & ~(size_t)255;
    const size_t cbase = wbase + partial_floats * sizeof(float);
    const size_t all = cbase + counters * sizeof(uint32_t);
    qwg_group *g = new (std::nothrow) qwg_group();
    if (!g) return QWG_ERR_HIP;
    if (hipGetDevice(&g->device) != hipSuccess || hipMalloc(&g->dev_mem, all) != hipSuccess) {
        delete g;
        return QWG_ERR_HIP;
    }
    uint8_t *base = (uint8_t *)g->dev_mem;
    if (split) {
        size_t pf = 0, ct = 0;
        for (int i = 0; i < count; ++i) {
            if (probs[i].splits < 2) continue;
            probs[i].partial = (float *)(base + wbase) + pf;
            probs[i].counters = (uint32_t *)(base + cbase) + ct;
            pf += (size_t)probs[i].splits * probs[i].tiles * kTileRows;
            ct += (size_t)probs[i].tiles;
        }
    }
    // Counters start at zero; every run leaves them at zero again.
    if ((counters && hipMemset(base + cbase, 0, counters * sizeof(uint32_t)) != hipSuccess) ||
        hipMemcpy(base, probs.data(), pbytes, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(base + pbytes, map.data(), mbytes, hipMemcpyHostToDevice) != hipSuccess ||
        (tbytes && hipMemcpy(base + pbytes + mbytes, tile.data(), tbytes, hipMemcpyHostToDevice) !=
                       hipSuccess)) {
        (void)hipFree(g->dev_mem);
        delete g;
        return QWG_ERR_HIP;
    }
    g->fmt = fmt;
    g->layout = layout;
    g->grid = grid;
    g->args.problems = (const GemvArgs *)g->dev_mem;
    g->args.map = (const uint32_t *)(base + pbytes);
    g->args.tile = tbytes ? (const uint32_t *)(base + pbytes + mbytes) : nullptr;
    g->count = count;
    g->workgroups = (int)total;
    g->positions = (int)positions;
    g->max_nb = max_nb;
    g->split = split;
    g->waves = ssh.waves;
    g->ring = ssh.ring;
    g->cb_shape = cb_shape;
    g->mring = mstream ? mstream_ring() : 0;
    g->batch = batch;
    // One column per stage: a group has thousands of workgroups, and the
    // 8-wavefront two-column shape that helps short single launches measured
    // slower on the 155-product stream (us, one column / two): batch 2 151.5 /
    // 166.1, batch 4 167.0 / 185.7, batch 8 176.1 / 196.6. QWG_MFMA_COLS forces
    // 1 or 2 (tuning).
    static const int env_cols = env_int("QWG_MFMA_COLS", 0);
    g->cols = env_cols == 1 || env_cols == 2 ? env_cols : 1;
    *out = g;
    return QWG_OK;
}

}  // namespace

int qwg_group_create_q4k(const qwg_gemv_desc *descs, int count, qwg_group **out) {
    if (!descs || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP) return QWG_ERR_SHAPE;
    return group_create(QWG_FMT_Q4K, kLayoutRows, descs, count, nullptr, out);
}

int qwg_group_create_q4k_batched(const qwg_gemv_desc *descs, int count, int batch,
                                 qwg_group **out) {
    if (!descs || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP) return QWG_ERR_SHAPE;
    if (batch < 2 || batch > QWG_MAX_BATCH) return QWG_ERR_BATCH;
    return group_create(QWG_FMT_Q4K, kLayoutRows, descs, count, nullptr, out, batch);
}

int qwg_group_create_q4k_batched_tiled(const qwg_gemv_desc *descs, int count, int batch,
                                       qwg_group **out) {
    if (!descs || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP) return QWG_ERR_SHAPE;
    if (batch < 2 || batch > QWG_MAX_BATCH) return QWG_ERR_BATCH;
    return group_create(QWG_FMT_Q4K, kLayoutTiles, descs, count, nullptr, out, batch);
}

int qwg_group_create_q4k_tiled(const qwg_gemv_desc *descs, int count, qwg_group **out) {
    if (!descs || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP) return QWG_ERR_SHAPE;
    return group_create(QWG_FMT_Q4K, kLayoutTiles, descs, count, nullptr, out);
}

int qwg_group_create_iq3(const qwg_gemv_desc *descs, int count, const float *grid,
                         qwg_group **out) {
    if (!descs || !grid || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP) return QWG_ERR_SHAPE;
    if (!aligned(grid, 16)) return QWG_ERR_ALIGN;
    return group_create(QWG_FMT_IQ3, kLayoutRows, descs, count, grid, out);
}

int qwg_group_create_iq3_tiled(const qwg_gemv_desc *descs, int count, const float *grid,
                               qwg_group **out) {
    if (!descs || !grid || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP) return QWG_ERR_SHAPE;
    if (!aligned(grid, 16)) return QWG_ERR_ALIGN;
    return group_create(QWG_FMT_IQ3, kLayoutTiles, descs, count, grid, out);
}

int qwg_group_create_iq3s(const qwg_gemv_desc *descs, int count, const float *grid,
                          qwg_group **out) {
    if (!descs || !grid || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP) return QWG_ERR_SHAPE;
    if (!aligned(grid, 16)) return QWG_ERR_ALIGN;
    return group_create(QWG_FMT_IQ3_S, kLayoutRows, descs, count, grid, out);
}

int qwg_group_create_iq4xs(const qwg_gemv_desc *descs, int count, const float *table,
                           qwg_group **out) {
    if (!descs || !table || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP) return QWG_ERR_SHAPE;
    if (!aligned(table, 16)) return QWG_ERR_ALIGN;
    return group_create(QWG_FMT_IQ4_XS, kLayoutRows, descs, count, table, out);
}

int qwg_group_create_iq3s_tiled(const qwg_gemv_desc *descs, int count, const float *grid,
                                qwg_group **out) {
    if (!descs || !grid || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP) return QWG_ERR_SHAPE;
    if (!aligned(grid, 16)) return QWG_ERR_ALIGN;
    return group_create(QWG_FMT_IQ3_S, kLayoutTiles, descs, count, grid, out);
}

int qwg_group_create_iq4xs_tiled(const qwg_gemv_desc *descs, int count, const float *table,
                                 qwg_group **out) {
    if (!descs || !table || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP) return QWG_ERR_SHAPE;
    if (!aligned(table, 16)) return QWG_ERR_ALIGN;
    return group_create(QWG_FMT_IQ4_XS, kLayoutTiles, descs, count, table, out);
}

int qwg_group_run(const qwg_group *g, void *stream) {
    if (!g) return QWG_ERR_NULL;
    GemvArgs unused;
    fill_shape(unused, nullptr, nullptr, nullptr, nullptr, kQK, 1, kQ4kBytes);
    if (g->batch >= 2 && g->mring)
        return hip_status(launch_q4k_mstream(g->args, unused, g->positions, g->batch, g->mring,
                                             false, (hipStream_t)stream));
    if (g->batch >= 2)
        return hip_status(
            launch_q4k_mfma_group(g->args, g->positions, g->batch, g->cols,
                                  g->layout == kLayoutTiles, (hipStream_t)stream));
    if (codebook_format(g->fmt))
        return hip_status(launch_cb_stream(g->fmt, g->layout == kLayoutTiles, g->cb_shape,
                                           g->args, unused, g->grid, g->positions,
                                           (hipStream_t)stream));
    if (g->fmt == QWG_FMT_IQ3)
        return hip_status(launch_iq3_stream(g->args, unused, g->grid, g->positions,
                                            iq3_shape(true, 0), g->layout == kLayoutTiles,
                                            (hipStream_t)stream));
    if (use_stream_engine() || g->layout == kLayoutTiles)
        return hip_status(launch_q4k_stream(g->args, unused, g->positions, g->waves, g->ring,
                                            g->split, (hipStream_t)stream));
    return hip_status(launch_q4k_group(g->args, g->workgroups, g->max_nb, (hipStream_t)stream));
}

int qwg_group_workgroups(const qwg_group *g) { return g ? g->workgroups : -QWG_ERR_NULL; }

}  // extern "C"

// ------------------------------------------------------------------ layer chain

struct qwg_chain {
    int device;
    void *dev_mem;   // members, units, phases, fin, partial sums, counters, flags, error word
    uint32_t *counters;
    ChainArgs args;
    int count;
    int launch_phases;
};

namespace {

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

// Workgroups of a chain launch: one per compute unit, a multiple of 8 (the
// XCDs), at most 256 (one flag per poll lane word).
int chain_workgroups() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (cus > 256) cus = 256;
    return cus - cus % 8;
}

}  // namespace

extern "C" {

int qwg_chain_create_q4k(const qwg_gemv_desc *descs, int count, const int *phase_sizes,
                         int n_phases, qwg_chain **out) {
    if (!descs || !phase_sizes || !out) return QWG_ERR_NULL;
    *out = nullptr;
    if (count < 1 || count > QWG_MAX_GROUP || n_phases < 1 || n_phases > count)
        return QWG_ERR_SHAPE;
    std::vector<int> phase_of((size_t)count);
    {
        int k = 0;
        for (int p = 0; p < n_phases; ++p) {
            if (phase_sizes[p] < 1 || k + phase_sizes[p] > count) return QWG_ERR_SHAPE;
            for (int i = 0; i < phase_sizes[p]; ++i) phase_of[(size_t)k++] = p;
        }
        if (k != count) return QWG_ERR_SHAPE;
    }
    std::vector<ChainMember> mem((size_t)count);
    for (int i = 0; i < count; ++i) {
        const qwg_gemv_desc &d = descs[i];
        if (!d.y || !d.x || !d.w) return QWG_ERR_NULL;
        const int rc = check_gemv_shape(d.n_in, d.n_out);
        if (rc) return rc;
        if (!aligned(d.w, 16) || !aligned(d.x, 16) || !aligned(d.y, 4)) return QWG_ERR_ALIGN;
        ChainMember &m = mem[(size_t)i];
        m.w = (const uint8_t *)d.w;
        m.x = d.x;
        m.y = d.y;
        m.partial = nullptr;
        m.counters = nullptr;
        m.n_out = (int)d.n_out;
        m.nb = (int)(d.n_in / kQK);
        m.tiles = (int)((d.n_out + kTileRows - 1) / kTileRows);
        m.splits = 1;
        m.mode = kChainDirect;
        m.ll = nullptr;
        m.xll = nullptr;
        m.done = nullptr;
        m.xsplits = 0;
        m.xstride = 0;
        m.tag = 0;
        m.xtag = 0;
        m.pad = 0;
    }
    // A member's activations may be the output of a member of an earlier phase
    // (read after that phase completed); they must not overlap an output of
    // the same phase.
    std::vector<bool> wired((size_t)count, false);
    for (int i = 0; i < count; ++i)
        for (int j = 0; j < count; ++j) {
            if (!overlaps(descs[j].x, (size_t)descs[j].n_in * 4, descs[i].y, (size_t)descs[i].n_out * 4))
                continue;
            if (phase_of[(size_t)i] >= phase_of[(size_t)j]) {
                if (phase_of[(size_t)i] == phase_of[(size_t)j]) return QWG_ERR_SHAPE;
                continue;   // written after it was read
            }
            wired[(size_t)i] = true;
        }
    // Tagged ordering (done words per tile, activations as tagged rows) needs
    // every activation read from the chain inside one earlier member's output,
    // and no output overlapping another output or an activation read in an
    // earlier phase (no phase may write what an earlier one still reads, since
    // workgroups no longer finish phases together). Otherwise the launch keeps
    // a flag barrier per phase. QWG_CHAIN_TAGGED=0 forces the barriers (A/B).
    const char *env_tg = getenv("QWG_CHAIN_TAGGED");
    bool dataflow = !(env_tg && env_tg[0] == '0');
    std::vector<int> producer((size_t)count, -1);
    for (int j = 0; j < count && dataflow; ++j) {
        const uintptr_t x0 = (uintptr_t)descs[j].x, x1 = x0 + (uintptr_t)descs[j].n_in * 4;
        for (int i = 0; i < count; ++i) {
            if (!overlaps(descs[j].x, (size_t)descs[j].n_in * 4, descs[i].y, (size_t)descs[i].n_out * 4))
                continue;
            const uintptr_t y0 = (uintptr_t)descs[i].y, y1 = y0 + (uintptr_t)descs[i].n_out * 4;
            if (phase_of[(size_t)i] < phase_of[(size_t)j] && y0 <= x0 && x1 <= y1 &&
                (x0 - y0) % 4 == 0 && producer[(size_t)j] < 0)
                producer[(size_t)j] = i;
            else
                dataflow = false;   // written after it was read, partly inside, or two producers
        }
    }
    for (int i = 0; i < count && dataflow; ++i)
        for (int k = i + 1; k < count; ++k)
            if (overlaps(descs[i].y, (size_t)descs[i].n_out * 4, descs[k].y, (size_t)descs[k].n_out * 4)) {
                dataflow = false;
                break;
            }
    const int nwg = chain_workgroups();
    if (nwg < 8) return QWG_ERR_HIP;
    const int64_t Q = (int64_t)nwg * kChainQuads;
    // Units: per phase a workgroup takes one chunk of C = 4 L consecutive
    // super-block columns of one 64-row tile of one member, L = 1 or 2 columns
    // for each of its four quads, whose sums meet in LDS; a tile's chunks are
    // its splits. L = 1 when the phase's chunks then fit the workgroups (more
    // of the chip computes each phase), else 2. Split partial sums meet in
    // split order: tagged launches let the consumers add a producer's partials
    // (tagged rows) and the launch's end finish y; barrier launches finish a
    // consumed member's tiles at once through a counter (wired), the others at
    // the end (deferred). A phase with more chunks than workgroups runs as
    // several launch phases of which only the first waits for the previous
    // phase.
    std::vector<uint32_t> units, phases, fin;
    size_t partial_floats = 0, counters = 0;
    int launch_phases = 0;
    int first = 0;
    // tagged launches: done words of every (tile, split) of every phase but the last
    std::vector<int64_t> done_off((size_t)count, -1), phase_done_off((size_t)n_phases, 0),
        phase_done_n((size_t)n_phases, 0);
    int64_t done_words = 0;
    for (int p = 0; p < n_phases; ++p) {
        const int last = first + phase_sizes[p];
        int L = 1;
        {
            int64_t chunks = 0;
            for (int i = first; i < last; ++i)
                chunks += (int64_t)mem[(size_t)i].tiles * ((mem[(size_t)i].nb + kChainQuads - 1) / kChainQuads);
            if (chunks > nwg) L = kChainMaxSteps;
        }
        const int C = kChainQuads * L;
        std::vector<std::array<uint32_t, 3>> list;   // (member, tile, split)
        phase_done_off[(size_t)p] = done_words;
        for (int i = first; i < last; ++i) {
            ChainMember &m = mem[(size_t)i];
            m.splits = (m.nb + C - 1) / C;
            if (dataflow && p + 1 < n_phases) {
                done_off[(size_t)i] = done_words;
                done_words += (int64_t)m.tiles * m.splits;
            }
            if (m.splits > 1) {
                // tagged launches: a consumed member's partials are its tagged
                // rows; every split member's y is finished at the end
                m.mode = !dataflow && wired[(size_t)i] ? kChainWired : kChainDeferred;
                if (!(dataflow && wired[(size_t)i]))
                    partial_floats += (size_t)m.splits * m.tiles * kTileRows;
                if (m.mode == kChainWired) counters += (size_t)m.tiles;
            }
            for (int t = 0; t < m.tiles; ++t) {
                for (int sp = 0; sp < m.splits; ++sp)
                    list.push_back({(uint32_t)i, (uint32_t)t, (uint32_t)sp});
                if (m.mode == kChainDeferred) {
                    fin.push_back((uint32_t)i);
                    fin.push_back((uint32_t)t);
                }
            }
        }
        for (size_t c0 = 0; c0 < list.size(); c0 += (size_t)nwg) {
            const size_t row = units.size();
            units.resize(row + (size_t)Q * 4, 0u);
            for (int64_t k = 0; k < Q; ++k) units[row + (size_t)k * 4] = kNoItem;
            for (size_t k = c0; k < std::min(list.size(), c0 + (size_t)nwg); ++k) {
                const int64_t wgi = (int64_t)(k - c0);
                const ChainMember &m = mem[(size_t)list[k][0]];
                const int sp = (int)list[k][2];
                for (int q = 0; q < kChainQuads; ++q) {
                    const int b0 = sp * C + q * L;
                    if (b0 >= m.nb) break;
                    const int nblk = std::min(L, m.nb - b0);
                    uint32_t *e = &units[row + (size_t)(wgi * kChainQuads + q) * 4];
                    e[0] = list[k][0];
                    e[1] = list[k][1];
                    e[2] = (uint32_t)b0 | (uint32_t)nblk << 8 | (uint32_t)sp << 16;
                    e[3] = 0u;
                }
            }
            const bool waits = p > 0 && c0 == 0;
            phases.push_back((uint32_t)L);
            if (dataflow) {
                // the done words of logical phase p - 1, tagged base + p
                phases.push_back(waits ? (uint32_t)p : 0u);
                phases.push_back(waits ? (uint32_t)phase_done_n[(size_t)(p - 1)] : 0u);
                phases.push_back(waits ? (uint32_t)phase_done_off[(size_t)(p - 1)] : 0u);
            } else {
                phases.push_back(waits ? 1u : 0u);
                phases.push_back(0u);
                phases.push_back(0u);
            }
            ++launch_phases;
        }
        phase_done_n[(size_t)p] = done_words - phase_done_off[(size_t)p];
        first = last;
    }
    if (launch_phases > (1 << 20) || fin.size() / 2 > (size_t)INT32_MAX) return QWG_ERR_SHAPE;
    // tagged rows of the producers' outputs: [splits][n_out] each
    std::vector<int64_t> ll_off((size_t)count, -1);
    int64_t ll_rows = 0;
    if (dataflow)
        for (int j = 0; j < count; ++j) {
            const int i = producer[(size_t)j];
            if (i < 0 || ll_off[(size_t)i] >= 0) continue;
            ll_off[(size_t)i] = ll_rows;
            ll_rows += (int64_t)mem[(size_t)i].splits * descs[i].n_out;
        }
    // device memory
    auto align256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t off_members = 0;
    const size_t off_units = align256(off_members + sizeof(ChainMember) * mem.size());
    const size_t off_phases = align256(off_units + sizeof(uint32_t) * units.size());
    const size_t off_fin = align256(off_phases + sizeof(uint32_t) * phases.size());
    const size_t off_partial = align256(off_fin + sizeof(uint32_t) * fin.size());
    const size_t off_counters = align256(off_partial + sizeof(float) * partial_floats);
    const size_t off_ll = align256(off_counters + sizeof(uint32_t) * counters);
    const size_t off_done = align256(off_ll + sizeof(uint64_t) * (size_t)ll_rows);
    const size_t off_flags = align256(off_done + sizeof(uint64_t) * (size_t)done_words);
    const size_t off_err = align256(off_flags + sizeof(uint32_t) * kFlagCopies * kFlagCopyWords);
    const size_t all = off_err + 256;
    qwg_chain *ch = new (std::nothrow) qwg_chain();
    if (!ch) return QWG_ERR_HIP;
    if (hipGetDevice(&ch->device) != hipSuccess || hipMalloc(&ch->dev_mem, all) != hipSuccess) {
        delete ch;
        return QWG_ERR_HIP;
    }
    uint8_t *base = (uint8_t *)ch->dev_mem;
    {
        size_t pf = 0, ct = 0;
        for (size_t i = 0; i < mem.size(); ++i) {
            ChainMember &m = mem[i];
            if (m.splits < 2 || (dataflow && ll_off[i] >= 0)) continue;
            m.partial = (float *)(base + off_partial) + pf;
            pf += (size_t)m.splits * m.tiles * kTileRows;
            if (m.mode == kChainWired) {
                m.counters = (uint32_t *)(base + off_counters) + ct;
                ct += (size_t)m.tiles;
            }
        }
        // Tags: a producer of logical phase P tags its rows base + P + 1 (the
        // run's base grows by the launch-phase count, at least the number of
        // logical phases, so consecutive runs never share a tag).
        uint64_t *ll = (uint64_t *)(base + off_ll);
        uint64_t *dw = (uint64_t *)(base + off_done);
        for (int i = 0; i < count; ++i) {
            mem[(size_t)i].tag = phase_of[(size_t)i] + 1;
            if (ll_off[(size_t)i] >= 0) mem[(size_t)i].ll = ll + ll_off[(size_t)i];
            if (done_off[(size_t)i] >= 0) mem[(size_t)i].done = dw + done_off[(size_t)i];
        }
        for (int j = 0; j < count; ++j) {
            const int i = producer[(size_t)j];
            if (!dataflow || i < 0) continue;
            mem[(size_t)j].xll = mem[(size_t)i].ll + ((const float *)descs[j].x - (const float *)descs[i].y);
            mem[(size_t)j].xtag = mem[(size_t)i].tag;
            mem[(size_t)j].xsplits = mem[(size_t)i].splits;
            mem[(size_t)j].xstride = mem[(size_t)i].n_out;
        }
    }
    // Counters, tagged rows and done words (tag 0: never a run's), flags and
    // the error word start at zero; every run leaves the counters at zero and
    // all flags equal.
    if (hipMemset(base + off_counters, 0, off_err + 256 - off_counters) != hipSuccess ||
        hipMemcpy(base + off_members, mem.data(), sizeof(ChainMember) * mem.size(),
                  hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(base + off_units, units.data(), sizeof(uint32_t) * units.size(),
                  hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(base + off_phases, phases.data(), sizeof(uint32_t) * phases.size(),
                  hipMemcpyHostToDevice) != hipSuccess ||
        (!fin.empty() && hipMemcpy(base + off_fin, fin.data(), sizeof(uint32_t) * fin.size(),
                                   hipMemcpyHostToDevice) != hipSuccess)) {
        (void)hipFree(ch->dev_mem);
        delete ch;
        return QWG_ERR_HIP;
    }
    ch->counters = (uint32_t *)(base + off_counters);
    ch->args.members = (const ChainMember *)(base + off_members);
    ch->args.units = (const uint32_t *)(base + off_units);
    ch->args.phases = (const uint32_t *)(base + off_phases);
    ch->args.fin = (const uint32_t *)(base + off_fin);
    ch->args.flags = (uint32_t *)(base + off_flags);
    ch->args.err = (uint32_t *)(base + off_err);
    ch->args.nphases = launch_phases;
    ch->args.nfin = (int)(fin.size() / 2);
    ch->args.done = (const uint64_t *)(base + off_done);
    ch->args.nwg = nwg;
    ch->args.tagged = dataflow ? 1 : 0;
    ch->count = count;
    ch->launch_phases = launch_phases;
    *out = ch;
    return QWG_OK;
}

int qwg_chain_run(const qwg_chain *c, void *stream) {
    if (!c) return QWG_ERR_NULL;
    return hip_status(launch_q4k_chain(c->args, (hipStream_t)stream));
}

int qwg_chain_phases(const qwg_chain *c) { return c ? c->launch_phases : -QWG_ERR_NULL; }

int qwg_chain_tagged(const qwg_chain *c) { return c ? c->args.tagged : -QWG_ERR_NULL; }

int qwg_chain_status(qwg_chain *c) {
    if (!c) return QWG_ERR_NULL;
    if (hipDeviceSynchronize() != hipSuccess) return QWG_ERR_HIP;
    uint32_t err = 0;
    if (hipMemcpy(&err, c->args.err, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess)
        return QWG_ERR_HIP;
    if (err == 0) return QWG_OK;
    // A wait gave up: tile counters, tagged rows, done words, flags and the
    // error word are re-armed (they lie back to back, the counters first; the
    // flags restart at zero, so no tagged word may keep a tag of the run that
    // gave up).
    if (hipMemset(c->counters, 0, (uint8_t *)c->args.err + sizeof(uint32_t) - (uint8_t *)c->counters) !=
        hipSuccess)
        return QWG_ERR_HIP;
    return QWG_ERR_TIMEOUT;
}

int qwg_chain_destroy(qwg_chain *c) {
    if (!c) return QWG_OK;
    const hipError_t e = hipFree(c->dev_mem);
    delete c;
    return hip_status(e);
}

int qwg_group_destroy(qwg_group *g) {
    if (!g) return QWG_OK;
    const hipError_t e = hipFree(g->dev_mem);
    delete g;
    return hip_status(e);
}

}  // extern "C"
