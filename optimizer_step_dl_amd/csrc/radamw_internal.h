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
// buckets, 4-read/3-write streams): many small single-tile workgroups,
// dispatched in tile order, keep the tiles in flight within a narrow address
// window; 64 lanes x 1 chunk beat 2-4 chunks per lane, 128- or 256-lane
// workgroups, grid-stride loops and persistent pipelined waves by 5-30%
// (with the occupancy cap below, 6.5-6.7 TB/s).
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

// Occupancy caps.  A CU of gfx950 has 160 KiB of LDS and holds up to 32
// waves.  The streaming kernels use (almost) no LDS, so by default a CU
// fills with 32 single-wave update workgroups, each with a whole tile of
// every stream in flight.  That is more than HBM serves best: on MI355X
// (2^28-element buckets, every update variant: FP32 / 16-bit gradients,
// AdamW / AMSGrad, steady / first step, with and without a model copy)
// throughput is highest when a CU holds about 64 KiB of tile traffic (reads
// plus writes), i.e. 7-14 workgroups, at 6.45-6.76 TB/s depending on the
// box, against 6.0-6.3 TB/s at full occupancy.  Budgets of 60-72 KiB are
// within 1% of one another for AdamW; 64 KiB was never worse than 72 KiB
// on two boxes and up to 1.9% better for AMSGrad and first steps; 56 KiB
// and below starve the memory system (5.5-6.3 TB/s).  The cap is applied
// by reserving LDS at launch that the kernels never touch.
constexpr int64_t LDS_PER_CU = 160 * 1024;
constexpr int MAX_WAVES_PER_CU = 32;
#ifndef RADAMW_CU_INFLIGHT_KIB
#define RADAMW_CU_INFLIGHT_KIB 64
#endif
constexpr int64_t UPDATE_CU_INFLIGHT_BYTES = int64_t(RADAMW_CU_INFLIGHT_KIB) * 1024;

// Dynamic LDS that, together with a kernel's `static_bytes` of static LDS,
// lets exactly `cap` workgroups reside on one CU: the total is the largest
// multiple of the 512-byte allocation unit not above LDS_PER_CU / cap, which
// stays above LDS_PER_CU / (cap + 1) for every cap up to 17.
inline size_t lds_for_cap(int64_t cap, size_t static_bytes) {
    if (cap < 1) cap = 1;
    const size_t total = static_cast<size_t>(LDS_PER_CU / cap) & ~size_t(511);
    const size_t st = (static_bytes + 511) & ~size_t(511);
    return total > st ? total - st : 0;
}

// HBM bytes one element of an update moves: p, the gradient and (after the
// first step) m, v and v_max read; p, m, v, v_max and the optional 16-bit
// model copy written.
inline int64_t update_bytes_per_element(int gdt, bool amsgrad, bool first, bool copy) {
    int64_t b = 4 + (gdt == 0 ? 4 : 2) + 12;  // read p, g; write p, m, v
    if (!first) b += 8;                       // read m, v
    if (amsgrad) b += first ? 4 : 8;          // [read] and write v_max
    if (copy) b += 2;
    return b;
}

// The LDS reservation of a streaming launch of single-wave workgroups with
// no static LDS, each moving `bytes_per_element` per element of a
// UPDATE_TILE_ELEMS tile: the largest number of resident workgroups whose
// tiles stay within UPDATE_CU_INFLIGHT_BYTES.
inline size_t stream_lds_reservation(int64_t bytes_per_element) {
    const int64_t cap = UPDATE_CU_INFLIGHT_BYTES / (bytes_per_element * UPDATE_TILE_ELEMS);
    return cap >= MAX_WAVES_PER_CU ? 0 : lds_for_cap(cap, 0);
}

inline size_t update_lds_reservation(int gdt, bool amsgrad, bool first, bool copy) {
    return stream_lds_reservation(update_bytes_per_element(gdt, amsgrad, first, copy));
}

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
// FP32 analysis keeps 16 KiB in flight per workgroup (256 lanes x 4
// chunks); on MI355X it read fastest with 4 resident workgroups per CU (7.1
// against 6.9 TB/s at the full 8).  The 16-bit analysis spends more ALU per
// byte (8 binary64 FMAs per 16-byte chunk) and needs every wave it can get
// (capping it cost up to 35%), so it runs uncapped.
constexpr int STATS_F32_WG_PER_CU = 4;
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
// bound (<= 0: no clipping); and, when `done` is set, the word of host
// memory mapped for the device to which it writes `seq` once the report
// and the decision are visible to the host.
struct DecideArgs {
    double gradient_scale;
    double max_grad_norm;
    uint32_t *done = nullptr;
    uint32_t seq = 0;
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
// copy: some segment of the table writes a model copy.
hipError_t launch_update_table(const SegDesc *segs_dev, const int64_t *tile_prefix_dev,
                               const int32_t *coarse_dev, int32_t nseg, int64_t total_tiles,
                               const Coefs &c, const Decision *dec, int gdt, bool amsgrad, bool first,
                               bool copy, int grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop);
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

// The streaming probe (measurement only): nr FP32 read streams and nw write
// streams of `chunks` 16-byte chunks each; out[0] is the sink of a
// read-only probe, stored to only where a sum equals sink_key (a NaN).
struct ProbeArgs {
    const float *in[5];
    float *out[4];
    int64_t chunks;
    float sink_key;
};
// cap_per_cu: resident workgroups per CU (1..32), or 0 for the update's rule
// (about UPDATE_CU_INFLIGHT_BYTES of tile traffic per CU).
hipError_t launch_stream_probe(const ProbeArgs &a, int nr, int nw, int cap_per_cu, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop);

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
