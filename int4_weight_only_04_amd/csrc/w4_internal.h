// Internal declarations shared by the host-side ABI code and the HIP kernels
// of the INT4 weight-only GEMV library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace w4i {

constexpr int kTileRows = 4;          // rows per packed tile (W4T4 layout)
constexpr int kBlockThreads = 256;    // 4 waves of 64 lanes
constexpr int kWavesPerBlock = kBlockThreads / 64;
constexpr int64_t kMaxK = 32768;      // x[k] is staged whole in LDS (64 KiB)
constexpr int kArgmaxMaxBlocks = 4096;
constexpr size_t kArgmaxHeaderBytes = 256;  // counter lives here
constexpr size_t kArgmaxWorkspaceBytes = kArgmaxHeaderBytes + 8 * (size_t)kArgmaxMaxBlocks;

enum Epilogue : int32_t {
    kEpiPlain = 0,   // y fp32
    kEpiArgmax = 1,  // y fp32 + lowest-index argmax
    kEpiGateUp = 2,  // h fp16 = silu(gate) * up
};

struct GemvCall {
    const void* pw;      // packed weights (device)
    const void* ps;      // packed scales (device)
    const void* x;       // fp16 [k] (device)
    void* out;           // fp32 [n] or fp16 [n/2] (device)
    int32_t* argmax;     // device, argmax epilogue only
    void* ws;            // device workspace, argmax epilogue only
    int64_t n;           // logical rows (gate/up: 2I)
    int64_t k;
    int32_t group;
    int32_t epi;
};

// Launch one GEMV on `stream` (shape already validated by the caller).
hipError_t launch_gemv(const GemvCall& call, hipStream_t stream);

// Resolve the launch's device queries (residency) ahead of a graph capture.
hipError_t prepare_gemv(const GemvCall& call);

// Number of W4T4 tiles of an n-row matrix in the given epilogue's layout.
inline int64_t tiles_for(int64_t n, bool gateup)
{
    if (gateup) return 2 * ((n / 2 + kTileRows - 1) / kTileRows);
    return (n + kTileRows - 1) / kTileRows;
}

}  // namespace w4i
