// C ABI of libqwg (declared in include/qwg.h): argument validation, work
// decomposition and launch. Every check runs on the host before any HIP call,
// so a rejected call touches neither the device nor the output buffers.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/qwg.h"
#include "qwg_internal.h"

using namespace qwg;

namespace {

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_gemv_shape(int64_t n_in, int64_t n_out) {
    if (n_in < kQK || n_in > QWG_MAX_N_IN || n_in % kQK) return QWG_ERR_SHAPE;
    if (n_out < 1 || n_out > QWG_MAX_N_OUT) return QWG_ERR_SHAPE;
    return QWG_OK;
}

// Workgroups wanted per launch: enough 4-wavefront groups to give every one of
// the 256 compute units several, so small matrices split their rows' block
// ranges rather than idle most of the chip. QWG_TARGET_WGS overrides it (tuning).
int target_workgroups() {
    static int v = [] {
        const char *e = getenv("QWG_TARGET_WGS");
        int t = e ? atoi(e) : 0;
        return t > 0 ? t : 2048;
    }();
    return v;
}

int choose_splits(int tiles, int nb) {
    int s = (target_workgroups() + tiles - 1) / tiles;
    if (s > nb) s = nb;
    if (s < 1) s = 1;
    return s;
}

// Split-sum workspace, one per (device, stream): partial sums [splits][batch]
// [tiles*64] fp32 followed by one counter per tile. Sized for the largest use:
// splits > 1 only when tiles < target (so splits*tiles < 2*target), times the
// batch and 64 rows, plus counters.
struct Workspace {
    float *partial = nullptr;
    uint32_t *counters = nullptr;
};

size_t workspace_partial_floats() { return (size_t)2 * target_workgroups() * QWG_MAX_BATCH * kTileRows; }
size_t workspace_counters() { return (size_t)target_workgroups(); }

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

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
    const size_t pbytes = workspace_partial_floats() * sizeof(float);
    const size_t cbytes = workspace_counters() * sizeof(uint32_t);
    void *mem = nullptr;
    if (hipMalloc(&mem, pbytes + cbytes) != hipSuccess) return QWG_ERR_HIP;
    // Counters start at zero; every launch leaves them at zero again.
    if (hipMemset((uint8_t *)mem + pbytes, 0, cbytes) != hipSuccess) {
        (void)hipFree(mem);
        return QWG_ERR_HIP;
    }
    Workspace ws;
    ws.partial = (float *)mem;
    ws.counters = (uint32_t *)((uint8_t *)mem + pbytes);
    g_ws.emplace(key, ws);
    *out = ws;
    return QWG_OK;
}

int fill_gemv_args(GemvArgs &a, const void *w, const float *x, const float *grid, float *y,
                   int64_t n_in, int64_t n_out, int block_bytes, int batch, hipStream_t stream) {
    a.w = (const uint8_t *)w;
    a.x = x;
    a.grid = grid;
    a.y = y;
    a.n_in = (int)n_in;
    a.n_out = (int)n_out;
    a.nb = (int)(n_in / kQK);
    a.row_bytes = (int64_t)a.nb * block_bytes;
    a.tiles = (int)((n_out + kTileRows - 1) / kTileRows);
    a.splits = choose_splits(a.tiles, a.nb);
    a.partial = nullptr;
    a.counters = nullptr;
    if (a.splits > 1) {
        Workspace ws;
        int rc = get_workspace(stream, &ws);
        if (rc != QWG_OK) return rc;
        if ((size_t)a.splits * batch * a.tiles * kTileRows > workspace_partial_floats() ||
            (size_t)a.tiles > workspace_counters())
            return QWG_ERR_SHAPE;  // unreachable by construction of choose_splits
        a.partial = ws.partial;
        a.counters = ws.counters;
    }
    return QWG_OK;
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
        default: return "unknown status";
    }
}

int64_t qwg_row_bytes(int fmt, int64_t n_in) {
    if (fmt != QWG_FMT_Q4K && fmt != QWG_FMT_IQ3) return -QWG_ERR_FORMAT;
    if (n_in <= 0 || n_in % kQK) return -QWG_ERR_SHAPE;
    return (n_in / kQK) * (fmt == QWG_FMT_Q4K ? kQ4kBytes : kIq3Bytes);
}

int qwg_plan_splits(int fmt, int64_t n_in, int64_t n_out) {
    if (fmt != QWG_FMT_Q4K && fmt != QWG_FMT_IQ3) return -QWG_ERR_FORMAT;
    int rc = check_gemv_shape(n_in, n_out);
    if (rc) return -rc;
    return choose_splits((int)((n_out + kTileRows - 1) / kTileRows), (int)(n_in / kQK));
}

int qwg_dequant_q4k(const void *src, float *dst, int64_t n, void *stream) {
    if (!src || !dst) return QWG_ERR_NULL;
    if (n <= 0 || n % kQK) return QWG_ERR_SHAPE;
    if (!aligned(src, 16) || !aligned(dst, 16)) return QWG_ERR_ALIGN;
    return hip_status(launch_q4k_dequant((const uint8_t *)src, dst, n / kQK, (hipStream_t)stream));
}

int qwg_dequant_iq3(const void *src, const float *grid, float *dst, int64_t n, void *stream) {
    if (!src || !grid || !dst) return QWG_ERR_NULL;
    if (n <= 0 || n % kQK) return QWG_ERR_SHAPE;
    if (!aligned(src, 2) || !aligned(grid, 16) || !aligned(dst, 16)) return QWG_ERR_ALIGN;
    return hip_status(
        launch_iq3_dequant((const uint8_t *)src, grid, dst, n / kQK, (hipStream_t)stream));
}

int qwg_gemm_q4k(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out, int batch,
                 void *stream) {
    if (!y || !x || !w) return QWG_ERR_NULL;
    int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (batch < 1 || batch > QWG_MAX_BATCH) return QWG_ERR_BATCH;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return QWG_ERR_ALIGN;
    GemvArgs a;
    rc = fill_gemv_args(a, w, x, nullptr, y, n_in, n_out, kQ4kBytes, batch, (hipStream_t)stream);
    if (rc) return rc;
    return hip_status(launch_q4k_gemv(a, batch, (hipStream_t)stream));
}

int qwg_gemv_q4k(float *y, const float *x, const void *w, int64_t n_in, int64_t n_out,
                 void *stream) {
    return qwg_gemm_q4k(y, x, w, n_in, n_out, 1, stream);
}

int qwg_gemv_iq3(float *y, const float *x, const void *w, const float *grid, int64_t n_in,
                 int64_t n_out, void *stream) {
    if (!y || !x || !w || !grid) return QWG_ERR_NULL;
    int rc = check_gemv_shape(n_in, n_out);
    if (rc) return rc;
    if (!aligned(w, 2) || !aligned(x, 16) || !aligned(grid, 16) || !aligned(y, 4))
        return QWG_ERR_ALIGN;
    GemvArgs a;
    rc = fill_gemv_args(a, w, x, grid, y, n_in, n_out, kIq3Bytes, 1, (hipStream_t)stream);
    if (rc) return rc;
    return hip_status(launch_iq3_gemv(a, (hipStream_t)stream));
}

}  // extern "C"
