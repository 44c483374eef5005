// radamw_probe.hip -- the streaming ceiling of the update's access pattern
// on gfx950, for measurement only (not part of the method).
//
// The update moves 4 reads + 3 writes (AdamW, FP32 gradient), 5 + 4
// (AMSGrad) or 2 + 3 (first step) four-byte streams per element.  This
// kernel moves NR read streams and NW write streams with the update's
// geometry -- one wave64 workgroup per 256-element tile, one 16-byte chunk
// per lane and stream, every load issued before any store, nontemporal
// dwordx4 loads and stores, and the same LDS-reservation occupancy rule
// applied to its own bytes per element -- but with one add per stream in
// place of the optimizer's arithmetic.  Its bandwidth is what the memory
// system gives this pattern, the figure the update kernel is compared with.
//
// out[w][i] = ((in[0][i] + in[1][i]) + ...) + w, the empty sum being 0.
// With no write stream the sum is stored only where it equals `sink_key`, a
// runtime value no sum reaches (the host passes a NaN, which compares
// unequal to everything), so the loads stay live and nothing is written.
#include "radamw_internal.h"

#include <hip/hip_ext.h>

namespace radamw {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int PROBE_BLOCK = 64;

template <int NR, int NW>
__global__ __launch_bounds__(PROBE_BLOCK) void stream_probe(ProbeArgs a) {
    const int64_t k = int64_t(blockIdx.x) * PROBE_BLOCK + threadIdx.x;
    if (k >= a.chunks) return;
    f32x4 x[NR > 0 ? NR : 1];
#pragma unroll
    for (int r = 0; r < NR; ++r) x[r] = __builtin_nontemporal_load(gl(reinterpret_cast<const f32x4 *>(a.in[r]) + k));
    f32x4 s = f32x4(0.0f);
#pragma unroll
    for (int r = 0; r < NR; ++r) s = r == 0 ? x[0] : s + x[r];
    if constexpr (NW == 0) {
        if (s.x == a.sink_key) gl(a.out[0])[4 * k] = s.x;
    } else {
#pragma unroll
        for (int w = 0; w < NW; ++w)
            __builtin_nontemporal_store(s + f32x4(float(w)), gl(reinterpret_cast<f32x4 *>(a.out[w]) + k));
    }
}

template <int NR, int NW>
static hipError_t launch_probe_t(const ProbeArgs &a, int grid, size_t lds, hipStream_t st, hipEvent_t start,
                                 hipEvent_t stop) {
    hipExtLaunchKernelGGL((stream_probe<NR, NW>), dim3(grid), dim3(PROBE_BLOCK), lds, st, start, stop, 0, a);
    return hipGetLastError();
}

template <int NR>
static hipError_t launch_probe_r(const ProbeArgs &a, int nw, int grid, size_t lds, hipStream_t st,
                                 hipEvent_t start, hipEvent_t stop) {
    switch (nw) {
    case 0: return launch_probe_t<NR, 0>(a, grid, lds, st, start, stop);
    case 1: return launch_probe_t<NR, 1>(a, grid, lds, st, start, stop);
    case 2: return launch_probe_t<NR, 2>(a, grid, lds, st, start, stop);
    case 3: return launch_probe_t<NR, 3>(a, grid, lds, st, start, stop);
    case 4: return launch_probe_t<NR, 4>(a, grid, lds, st, start, stop);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_stream_probe(const ProbeArgs &a, int nr, int nw, int cap_per_cu, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop) {
    const int64_t grid = (a.chunks + PROBE_BLOCK - 1) / PROBE_BLOCK;
    if (grid < 1 || grid > UPDATE_MAX_GRID) return hipErrorInvalidValue;
    const size_t lds = cap_per_cu > 0 ? (cap_per_cu >= MAX_WAVES_PER_CU ? 0 : lds_for_cap(cap_per_cu, 0))
                                      : stream_lds_reservation(4 * int64_t(nr + nw));
    const int g = static_cast<int>(grid);
    switch (nr) {
    case 0: return launch_probe_r<0>(a, nw, g, lds, stream, start, stop);
    case 1: return launch_probe_r<1>(a, nw, g, lds, stream, start, stop);
    case 2: return launch_probe_r<2>(a, nw, g, lds, stream, start, stop);
    case 3: return launch_probe_r<3>(a, nw, g, lds, stream, start, stop);
    case 4: return launch_probe_r<4>(a, nw, g, lds, stream, start, stop);
    case 5: return launch_probe_r<5>(a, nw, g, lds, stream, start, stop);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace radamw
