// q4_launch.hpp -- host launchers of the gfx950 kernels.  Arguments have
// already been validated by the C ABI layer (q4_api.hip); each launcher only
// picks a kernel configuration and enqueues it on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace q4 {

struct DeviceInfo {
    int cu_count;        // compute units of the current device
};

// Cached per-device facts (thread-safe, filled on first use of a device).
const DeviceInfo& device_info(int device);

// True when `device` (0 <= device < 64) is a gfx950 the kernels were built for.
bool device_usable(int device);

// Allows `kernel` `bytes` of dynamic LDS on the current device.  The setting
// is made once per device (bit d of `done` records device d); safe to call
// from several threads.
hipError_t allow_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done);

// A GEMM tile shape and the time (microseconds, measured at k = 2560) one
// round of it takes when every CU runs one tile; only the ratios matter.
struct TileChoice {
    int bm, bn;
    float round_us;
};

// Index of the shape in `tiles` whose estimated time -- rounds of tiles over
// the CUs times its round time -- is least for m rows and the column counts
// n[0..count) (ties to the earlier entry: list the larger tiles first).
// Large tiles move the fewest operand bytes per output; too few of them
// leave CUs idle.
inline int choose_tile(const TileChoice* tiles, int ntiles, int64_t m, int count,
                       const int64_t* n, int cu_count) {
    int best = 0;
    double best_us = 0.0;
    for (int c = 0; c < ntiles; ++c) {
        int64_t t = 0;
        for (int i = 0; i < count; ++i) t += (n[i] + tiles[c].bn - 1) / tiles[c].bn;
        t *= (m + tiles[c].bm - 1) / tiles[c].bm;
        const double us = (double)((t + cu_count - 1) / cu_count) * tiles[c].round_us;
        if (c == 0 || us < best_us) {
            best = c;
            best_us = us;
        }
    }
    return best;
}

hipError_t launch_quantize(const float* w, uint8_t* packed, uint16_t* scales,
                           int64_t n, int64_t k, hipStream_t stream);

hipError_t launch_gemv(const uint16_t* x, const uint8_t* packed,
                       const uint16_t* scales, float* y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream);

// count (1..8) matrices sharing x and k, 1 <= m <= 8; host arrays.
hipError_t launch_gemv_multi(const uint16_t* x, int64_t m, int64_t k, int count,
                             const uint8_t* const* packed, const uint16_t* const* scales,
                             float* const* y, const int64_t* n, hipStream_t stream);

// fp16 weights [n, k], 1 <= m <= 8.
hipError_t launch_gemv_f16(const uint16_t* x, const uint16_t* w, float* y, int64_t m,
                           int64_t n, int64_t k, hipStream_t stream);

// fp16 weights [n, k], any m (m <= 8 -> launch_gemv_f16).
hipError_t launch_gemm_f16(const uint16_t* x, const uint16_t* w, float* y, int64_t m,
                           int64_t n, int64_t k, hipStream_t stream);

// Lists of the fused m = 1 top-k GEMV for n rows (0 when k does not fit the
// streaming kernel), and its launch writing those lists to `partials`.
int64_t gemv1_topk_lists(int64_t n, int64_t k, int cu_count);
hipError_t launch_gemv1_topk(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                             int64_t n, int64_t k, uint64_t* partials, hipStream_t stream);

// LM-head product followed by the per-token top-k (1 <= topk <= 32).
size_t gemv_topk_workspace(int64_t m, int64_t n, int64_t k, int cu_count);
hipError_t launch_gemv_topk(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                            int64_t m, int64_t n, int64_t k, int topk, float* values,
                            int32_t* rows, void* workspace, hipStream_t stream);

// count (1..8) matrices sharing x and k, any m >= 1; host arrays.
hipError_t launch_gemm_multi(const uint16_t* x, int64_t m, int64_t k, int count,
                             const uint8_t* const* packed, const uint16_t* const* scales,
                             float* const* y, const int64_t* n, hipStream_t stream);

hipError_t launch_gemm(const uint16_t* x, const uint8_t* packed,
                       const uint16_t* scales, float* y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream);

// The GEMM's small-batch kernel (16-row tiles of 16 columns, K split over the
// waves of a tile) for count (1..8) matrices sharing x and k, 1 <= m <= 16.
hipError_t launch_gemm_small(const uint16_t* x, int count, const uint8_t* const* packed,
                             const uint16_t* const* scales, float* const* y, const int64_t* n,
                             int64_t m, int64_t k, hipStream_t stream);

// At 2 <= m <= 8, matrices of at most this many rows go to launch_gemm_small
// instead of the block-diagonal GEMV: one GEMV wave owns 16 rows and walks all
// of K, so a few thousand rows keep only a few hundred waves busy, each with
// a long serial chain of steps (k = 2560, n = 4096, m = 8: 10.8 us against
// 6.3 us for the GEMM's tiles, whose waves split K; from n = 8192 up the GEMV
// is as fast or faster).
constexpr int64_t kGemvTileRows = 4096;

}  // namespace q4
