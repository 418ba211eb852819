// Internal interface between the C-ABI layer (qwg_api.cpp) and the kernel
// translation units (q4k.hip, iq3.hip). Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qwg {

constexpr int kQK = 256;
constexpr int kQ4kBytes = 144;
constexpr int kIq3Bytes = 98;
constexpr int kTileRows = 64;  // one output row per lane of a wavefront

// One GEMV/GEMM problem as the kernels see it. `splits` workgroups share each
// 64-row tile, each summing a contiguous range of super-blocks; with
// splits > 1 they meet in `partial` ([splits][batch][tiles*64] fp32) and the
// last to arrive at `counters[tile]` adds the partial sums in split order.
struct GemvArgs {
    const uint8_t *w;
    const float *x;
    const float *grid;   // IQ3 only
    float *y;
    float *partial;
    uint32_t *counters;
    int64_t row_bytes;
    int n_in;
    int n_out;
    int nb;       // super-blocks per row
    int tiles;    // ceil(n_out / 64)
    int splits;   // 1..nb
};

// Launchers: return hipSuccess or the launch error.
hipError_t launch_q4k_dequant(const uint8_t *src, float *dst, int64_t nblocks, hipStream_t s);
hipError_t launch_iq3_dequant(const uint8_t *src, const float *grid, float *dst,
                              int64_t nblocks, hipStream_t s);
hipError_t launch_q4k_gemv(const GemvArgs &a, int batch, hipStream_t s);
hipError_t launch_iq3_gemv(const GemvArgs &a, hipStream_t s);

}  // namespace qwg
