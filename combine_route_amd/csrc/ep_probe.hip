// Access-pattern probes (include/ep_probe.h): the HBM patterns of the
// dispatch copy and the combine with routing, metadata and layout taken out,
// so the kernels' rates can be set against what this memory delivers on the
// same pattern. One wave moves one piece of one row; rows go through per-row
// buffer resources, so no access leaves its row.
#include "ep_probe.h"

#include <hip/hip_runtime.h>

#include "ep_device.h"

namespace ep {
namespace {

using dev::bload16;
using dev::bstore16;
using dev::row_rsrc;
using dev::u32x4;

constexpr int kVpl = 8;         // 16-byte vectors a lane holds per chunk
constexpr int kGatherRows = 8;  // rows loaded before folding
constexpr int kGatherCols = 2;  // 16-byte columns a lane per pass
constexpr int kLoad = 2;        // nt: loads stream past the caches
constexpr int kGatherStore = 2; // the combine's stores stream
constexpr int kCopyStore = 0;   // the copies' stores do not

// One instance per kind (EP_PROBE_*), so profiles name the pattern.
template <int KIND>
__global__ __launch_bounds__(1024) void ep_probe_kernel(ProbeArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t flat = (int64_t)blockIdx.x * (blockDim.x / kWave) +
                         dev::uniform(threadIdx.x / kWave);
    const int64_t row = flat / a.pieces;
    if (row >= a.rows)
        return;  // whole waves only
    const int piece = (int)(flat - row * a.pieces);
    const int row_vecs = (int)(a.row_bytes / 16u);
    const int piece_vecs = (row_vecs + a.pieces - 1) / a.pieces;
    const int vbeg = piece * piece_vecs;
    const int vend = min(row_vecs, vbeg + piece_vecs);

    // the row's map list: lane i < stride holds entry i; the list ends at the
    // first entry < 0
    int32_t ent = -1;
    int n = 0;
    if constexpr (KIND == EP_PROBE_FANOUT || KIND == EP_PROBE_GATHER) {
        ent = lane < a.stride ? a.map[row * a.stride + lane] : -1;
        const uint64_t neg = __ballot(ent < 0);
        n = neg ? (int)__builtin_ctzll(neg) : kWave;
        n = min(n, a.stride);
    }

    if constexpr (KIND == EP_PROBE_READ) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.src + row * a.row_bytes, a.row_bytes);
        uint32_t acc = 0;
        for (int v0 = vbeg; v0 < vend; v0 += kWave * kVpl) {
            u32x4 v[kVpl];
#pragma unroll
            for (int u = 0; u < kVpl; ++u) {
                const int vv = v0 + u * kWave + lane;
                v[u] = vv < vend ? bload16<kLoad>(rs, (uint32_t)vv * 16u) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < kVpl; ++u)
                acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1)
            acc ^= (uint32_t)__shfl_xor((int)acc, off);
        if (lane == 0)
            reinterpret_cast<uint32_t*>(a.dst)[flat] = acc;
        return;
    }
    if constexpr (KIND == EP_PROBE_WRITE) {
        const __amdgpu_buffer_rsrc_t rd = row_rsrc(a.dst + row * a.row_bytes, a.row_bytes);
        for (int vv = vbeg + lane; vv < vend; vv += kWave) {
            const u32x4 w = {(uint32_t)row, (uint32_t)vv, 0u, 0u};
            bstore16<kCopyStore>(w, rd, (uint32_t)vv * 16u);
        }
        return;
    }
    if constexpr (KIND == EP_PROBE_COPY || KIND == EP_PROBE_FANOUT) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(a.src + row * a.row_bytes, a.row_bytes);
        for (int v0 = vbeg; v0 < vend; v0 += kWave * kVpl) {
            u32x4 v[kVpl];
#pragma unroll
            for (int u = 0; u < kVpl; ++u) {
                const int vv = v0 + u * kWave + lane;
                if (vv < vend)
                    v[u] = bload16<kLoad>(rs, (uint32_t)vv * 16u);
            }
            const int nd = KIND == EP_PROBE_COPY ? 1 : n;
            for (int i = 0; i < nd; ++i) {
                int64_t d = row;
                if constexpr (KIND == EP_PROBE_FANOUT) {
                    d = __builtin_amdgcn_readlane(ent, i);
                    if (d >= a.map_rows)
                        continue;
                }
                const __amdgpu_buffer_rsrc_t rd = row_rsrc(a.dst + d * a.row_bytes, a.row_bytes);
#pragma unroll
                for (int u = 0; u < kVpl; ++u) {
                    const int vv = v0 + u * kWave + lane;
                    if (vv < vend)
                        bstore16<kCopyStore>(v[u], rd, (uint32_t)vv * 16u);
                }
            }
        }
        return;
    }
    if constexpr (KIND != EP_PROBE_GATHER)
        return;
    // EP_PROBE_GATHER: bf16 rows, FP32 sum in list order from the first row,
    // round to nearest even once
    const __amdgpu_buffer_rsrc_t rd = row_rsrc(a.dst + row * a.row_bytes, a.row_bytes);
    for (int v0 = vbeg; v0 < vend; v0 += kWave * kGatherCols) {
        // the sum starts at -0, the identity of IEEE addition (-0 + x = x)
        float acc[kGatherCols][8];
#pragma unroll
        for (int u = 0; u < kGatherCols; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[u][e] = -0.0f;
        for (int i0 = 0; i0 < n; i0 += kGatherRows) {
            u32x4 rows[kGatherCols][kGatherRows];
#pragma unroll
            for (int q = 0; q < kGatherRows; ++q) {
                if (i0 + q < n) {
                    int64_t s = __builtin_amdgcn_readlane(ent, i0 + q);
                    s = s < a.map_rows ? s : 0;  // out-of-range entries read row 0
                    const __amdgpu_buffer_rsrc_t rs =
                        row_rsrc(a.src + s * a.row_bytes, a.row_bytes);
#pragma unroll
                    for (int u = 0; u < kGatherCols; ++u) {
                        const int vv = v0 + u * kWave + lane;
                        if (vv < vend)
                            rows[u][q] = bload16<kLoad>(rs, (uint32_t)vv * 16u);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < kGatherRows; ++q) {
                if (i0 + q < n) {
#pragma unroll
                    for (int u = 0; u < kGatherCols; ++u) {
                        float f[8];
                        dev::widen<0>(rows[u][q], f);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[u][e] = acc[u][e] + f[e];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherCols; ++u) {
            const int vv = v0 + u * kWave + lane;
            if (vv < vend)
                bstore16<kGatherStore>(dev::narrow<0>(acc[u]), rd, (uint32_t)vv * 16u);
        }
    }
}

}  // namespace

hipError_t launch_probe(const ProbeArgs& a, int waves, hipStream_t s)
{
    const int64_t waves_total = a.rows * a.pieces;
    if (waves_total == 0)
        return hipSuccess;
    const dim3 block((unsigned)(waves * kWave));
    const dim3 grid((unsigned)((waves_total + waves - 1) / waves));
    switch (a.kind) {
    case EP_PROBE_READ: hipLaunchKernelGGL(ep_probe_kernel<EP_PROBE_READ>, grid, block, 0, s, a); break;
    case EP_PROBE_WRITE: hipLaunchKernelGGL(ep_probe_kernel<EP_PROBE_WRITE>, grid, block, 0, s, a); break;
    case EP_PROBE_COPY: hipLaunchKernelGGL(ep_probe_kernel<EP_PROBE_COPY>, grid, block, 0, s, a); break;
    case EP_PROBE_FANOUT: hipLaunchKernelGGL(ep_probe_kernel<EP_PROBE_FANOUT>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(ep_probe_kernel<EP_PROBE_GATHER>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace ep
