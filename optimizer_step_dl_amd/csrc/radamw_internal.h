// radamw_internal.h -- structures shared by the C-ABI layer (radamw_api.cpp)
// and the gfx950 kernels (radamw_update.hip, radamw_stats.hip).  Not part of
// the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace radamw {

// Workgroup shape of the update kernels: one wave64 per workgroup, each lane
// owning UPDATE_UNROLL 16-byte FP32 chunks (4 elements) of every stream per
// tile, and one tile per workgroup.  Measured on MI355X (2^28-element
// buckets, 4-read/3-write streams): many small single-tile workgroups keep
// the most independent requests in flight; 64 lanes x 1 chunk reached
// ~6.3-6.4 TB/s where 256 lanes x 4 chunks with a grid-stride loop reached
// ~5.6 TB/s.
#ifndef RADAMW_UPDATE_BLOCK
#define RADAMW_UPDATE_BLOCK 64
#endif
constexpr int UPDATE_BLOCK = RADAMW_UPDATE_BLOCK;
#ifndef RADAMW_UPDATE_UNROLL
#define RADAMW_UPDATE_UNROLL 1
#endif
constexpr int UPDATE_UNROLL = RADAMW_UPDATE_UNROLL;
constexpr int64_t UPDATE_TILE_CHUNKS = int64_t(UPDATE_BLOCK) * UPDATE_UNROLL;  // float4 chunks per tile
constexpr int64_t UPDATE_TILE_ELEMS = UPDATE_TILE_CHUNKS * 4;

// Multi-tensor launch policy.  On MI355X, back-to-back launches of large
// tensors pipeline with no visible gap, and a shared launch across large
// tensors held in separate allocations measured 7-10% slower than one
// launch per tensor; for small tensors one shared launch avoids a launch
// (and its gap) per tensor.  Tensors of at least this many elements are
// launched on their own, all smaller ones share one launch.
constexpr int64_t MULTI_SOLO_MIN = int64_t(1) << 22;

// Coarse index of the multi-tensor kernel: one entry per 2^10 tiles
// (256K elements), naming the segment that holds that tile.
constexpr int TABLE_COARSE_LOG2 = 10;
// A multi-tensor statistics launch indexes its rows the same way: coarse
// entry j names the gradient holding row j << STATS_COARSE_LOG2.
constexpr int STATS_COARSE_LOG2 = 8;

// Grid of the update kernels: exactly one workgroup per tile.  A launch may
// hold at most this many tiles (~5.5e11 elements, far beyond device memory).
constexpr int64_t UPDATE_MAX_GRID = 0x7fffffff;

// Statistics: 256-lane analysis workgroups, each lane loads STATS_UNROLL
// 16-byte chunks per pass; one record ("row") per workgroup.
constexpr int STATS_BLOCK = 256;
#ifndef RADAMW_STATS_UNROLL
#define RADAMW_STATS_UNROLL 4
#endif
constexpr int STATS_UNROLL = RADAMW_STATS_UNROLL;
#ifndef RADAMW_STATS_ROWS_CAP
#define RADAMW_STATS_ROWS_CAP 8192
#endif
constexpr int64_t STATS_ROWS_CAP = RADAMW_STATS_ROWS_CAP;  // records per tensor, at most
constexpr int MERGE_BLOCK = 1024;            // merge workgroup = fan-in
constexpr int64_t MERGE_FAN_IN = 1024;
constexpr int64_t STATS_MAX_ROWS = 4194304;  // accepted by the merge plan

enum GradType : int { G_F32 = 0, G_F16 = 1, G_BF16 = 2 };

// FP32 coefficients of one update, formed on the host in FP64 and cast.
struct Coefs {
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float inv_scale;   // +-1 / gradient_scale (sign carries maximize)
    float decay;       // 1 - lr * weight_decay
    float step_size;   // lr / (1 - beta1^t)
    float inv_bc2;     // 1 / (1 - beta2^t)
    float eps;
};

// One contiguous tensor as the kernels see it.  For an in-place update the
// *_out pointers equal the *_in pointers.  head is the number of leading
// elements handled by scalar code so that every stream is 16-byte aligned
// from element `head` on (0..3); head == -1 marks a segment whose streams
// are not mutually aligned, processed entirely by scalar code.  model, when
// model_kind is G_F16 or G_BF16, receives the updated parameters rounded to
// that 16-bit type (the model copy of an FP32-master optimizer).
struct SegDesc {
    const float *p_in;
    const void *g;
    const float *m_in;
    const float *v_in;
    const float *vmax_in;
    float *p_out;
    float *m_out;
    float *v_out;
    float *vmax_out;
    void *model;
    int64_t n;
    int64_t tile_begin;  // first tile of this segment in the launch's tile space
    int32_t head;
    int32_t model_kind;  // 0: no copy; G_F16 / G_BF16: copy dtype
};

// Tiles a segment occupies (0 for an empty segment).
__host__ __device__ inline int64_t segment_tiles(int64_t n, int32_t head) {
    if (n == 0) return 0;
    if (head < 0) return (n + UPDATE_TILE_ELEMS - 1) / UPDATE_TILE_ELEMS;
    int64_t body_chunks = (n - head) / 4;
    int64_t t = (body_chunks + UPDATE_TILE_CHUNKS - 1) / UPDATE_TILE_CHUNKS;
    return t < 1 ? 1 : t;
}

// 12-byte statistics record: w[0] | w[1] << 32 = binary64 sum of squares of
// finite values, w[2] = saturating non-finite count.
struct StatsRec {
    uint32_t w[3];
};

// The skip / clip decision of a fused step, taken on the device by the final
// merge so that the update kernels can be queued before the host has read
// the report back: skip != 0 when the report counts a non-finite value;
// otherwise inv_scale, given the sign of the kernel's own Coefs::inv_scale
// (maximize), replaces the update's unscale factor.
struct Decision {
    uint32_t skip;
    float inv_scale;  // (float)(1 / (gradient_scale / clip)), clip folded in
};
static_assert(sizeof(Decision) == 8 && offsetof(Decision, inv_scale) == 4,
              "the update kernels load a decision as two 32-bit words");

// What the final merge needs to decide: the caller's scale and the clip
// bound (<= 0: no clipping).
struct DecideArgs {
    double gradient_scale;
    double max_grad_norm;
};

// Global-address-space views of generic pointers.  Tensor pointers that
// reach a kernel through memory (the multi-tensor descriptor table) are
// generic to the compiler, which would then emit FLAT instructions; these
// casts make every stream access a global_load / global_store.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T *gl(const T *p) {
    return (const __attribute__((address_space(1))) T *)p;
}
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T *gl(T *p) {
    return (__attribute__((address_space(1))) T *)p;
}

// Launchers (host functions defined next to the kernels).  They return the
// hipError_t of the launch.
// start / stop (may be null) are recorded at the kernel's start and end
// (hipExtLaunchKernelGGL), for measurement.
// dec (device, may be null): a decision the kernels read before storing; a
// skip decision leaves every buffer unwritten, otherwise its inv_scale
// replaces c.inv_scale.
hipError_t launch_update_single(const SegDesc &seg, const Coefs &c, const Decision *dec, int gdt,
                                bool amsgrad, bool first, int grid, hipStream_t stream, hipEvent_t start,
                                hipEvent_t stop);
hipError_t launch_update_table(const SegDesc *segs_dev, const int64_t *tile_prefix_dev,
                               const int32_t *coarse_dev, int32_t nseg, int64_t total_tiles,
                               const Coefs &c, const Decision *dec, int gdt, bool amsgrad, bool first,
                               int grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop);
// One gradient of a multi-tensor statistics launch: its records are
// out[row_begin, row_begin + rows), laid out exactly as a single-tensor
// launch would write them.
struct StatsSeg {
    const void *g;
    int64_t n;
    int64_t row_begin;
    int32_t head;
    int32_t rows;
};

// The staged (unfused) baseline: 4 launches (5 with vmax != null); *launched
// receives how many were submitted.
hipError_t launch_staged(float *p, const void *g, int gdt, float *m, float *v, float *vmax, float *delta,
                         int64_t n, bool first, const Coefs &c, hipStream_t stream, int *launched);
hipError_t launch_analyze(const void *g, int gdt, int64_t n, int32_t head, int64_t rows,
                          StatsRec *out, hipStream_t stream);
hipError_t launch_analyze_table(const StatsSeg *segs_dev, const int32_t *coarse_dev, int64_t total_rows,
                                int gdt, StatsRec *out, hipStream_t stream);
hipError_t launch_merge(const StatsRec *in, int64_t nin, int64_t per_block, int64_t nblocks,
                        StatsRec *out, hipStream_t stream);
// The final merge of a fused step: one workgroup reduces all nin records,
// writes the report to `out` and the decision to dec_dev and dec_host.
hipError_t launch_merge_decide(const StatsRec *in, int64_t nin, StatsRec *out, Decision *dec_dev,
                               Decision *dec_host, const DecideArgs &a, hipStream_t stream);

}  // namespace radamw
