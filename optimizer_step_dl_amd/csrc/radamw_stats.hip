// radamw_stats.hip -- gradient statistics for gfx950: the read-only analysis
// pass and the fan-in-1024 merge.
//
// Page abbreviations: FA-ja = RUDA docs page "実験的なデバイス上の融合 AdamW /
// AMSGrad"; TR-zh = "训练与状态保存".
//
// The analysis pass (FA-ja "ネイティブ PyTorch ストレージと階層統計":
// analyze_gradient) reads a gradient once and writes one 12-byte record per
// workgroup: the FP64 sum of squares of the finite values and the count of
// non-finite ones.  The merges (merge_gradient_stats_chunks /
// merge_gradient_stats) reduce up to 1024 records per workgroup; a
// 1024-lane workgroup gives each lane one record, so fan-in equals the
// workgroup size (TR-zh "在 ruda:0 上进行原生 PyTorch 训练": fan-in 1024).
//
// No atomics anywhere: every lane accumulates a fixed set of elements in a
// fixed order, wave64 butterflies (__shfl_xor) and a fixed LDS pass finish
// the workgroup, so the same input gives the same bits on every run.
#include "radamw_internal.h"

namespace radamw {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Acc {
    double s[4];
    uint32_t bad;
};

__device__ __forceinline__ void acc_value(Acc &a, int slot, float x) {
    const bool finite = __builtin_isfinite(x);
    const double d = finite ? static_cast<double>(x) : 0.0;
    a.s[slot] = __builtin_fma(d, d, a.s[slot]);  // d*d is exact in binary64
    a.bad += finite ? 0u : 1u;
}

// A finite value: add its exact square (binary64) to slot `slot`.
__device__ __forceinline__ void acc_finite(Acc &a, int slot, float x) {
    const double d = static_cast<double>(x);
    a.s[slot] = __builtin_fma(d, d, a.s[slot]);
}

// For a 32-bit word holding two 16-bit values whose exponent field is `exp`
// (0x7f80 bfloat16, 0x7c00 binary16): bit 15 / bit 31 of the result is set
// exactly when the low / high value has an all-ones exponent (inf or NaN),
// since adding the field's lowest bit carries into the value's sign position
// only from all ones.
template <uint32_t EXP>
__device__ __forceinline__ uint32_t nonfinite_pairs(uint32_t w) {
    constexpr uint32_t field = EXP | (EXP << 16);
    constexpr uint32_t low_bit = (EXP & (~EXP + 1u)) | ((EXP & (~EXP + 1u)) << 16);
    return ((w & field) + low_bit) & 0x80008000u;
}

template <int GDT>
__device__ __forceinline__ void acc_chunk(Acc &a, const void *g, int64_t chunk) {
    if constexpr (GDT == G_F32) {
        const f32x4 x = __builtin_nontemporal_load(gl(reinterpret_cast<const f32x4 *>(g)) + chunk);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc_value(a, j, x[j]);
    } else {
        // 16-bit values: one integer test per word flags non-finite pairs;
        // clean words (the usual case) skip the per-value selects
        const u32x4 w = __builtin_nontemporal_load(gl(reinterpret_cast<const u32x4 *>(g)) + chunk);
        constexpr uint32_t EXP = GDT == G_F16 ? 0x7c00u : 0x7f80u;
        const uint32_t bad = nonfinite_pairs<EXP>(w[0]) | nonfinite_pairs<EXP>(w[1]) |
                             nonfinite_pairs<EXP>(w[2]) | nonfinite_pairs<EXP>(w[3]);
        if (bad == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (GDT == G_F16) {
                    acc_finite(a, j, static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j]))));
                    acc_finite(a, j, static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j] >> 16))));
                } else {
                    acc_finite(a, j, __builtin_bit_cast(float, w[j] << 16));
                    acc_finite(a, j, __builtin_bit_cast(float, w[j] & 0xffff0000u));
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (GDT == G_F16) {
                    acc_value(a, j, static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j]))));
                    acc_value(a, j, static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j] >> 16))));
                } else {
                    acc_value(a, j, __builtin_bit_cast(float, w[j] << 16));
                    acc_value(a, j, __builtin_bit_cast(float, w[j] & 0xffff0000u));
                }
            }
        }
    }
}

template <int GDT>
__device__ __forceinline__ float load_one(const void *g, int64_t e) {
    if constexpr (GDT == G_F32) return gl(static_cast<const float *>(g))[e];
    else if constexpr (GDT == G_F16) return static_cast<float>(gl(static_cast<const _Float16 *>(g))[e]);
    else return __builtin_bit_cast(float, uint32_t(gl(static_cast<const uint16_t *>(g))[e]) << 16);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ StatsRec write_record(StatsRec *out, double s, uint64_t count) {
    const uint64_t bits = __builtin_bit_cast(uint64_t, s);
    StatsRec r;
    r.w[0] = uint32_t(bits);
    r.w[1] = uint32_t(bits >> 32);
    r.w[2] = count > 0xffffffffull ? 0xffffffffu : uint32_t(count);
    out->w[0] = r.w[0];
    out->w[1] = r.w[1];
    out->w[2] = r.w[2];
    return r;
}

// Fixed-order workgroup reduction; thread 0 writes the record and returns
// it (other threads return an unspecified record).
template <int BLOCK>
__device__ __forceinline__ StatsRec block_finish(double s, uint64_t count, StatsRec *out) {
    constexpr int WAVES = BLOCK / 64;
    __shared__ double ws[WAVES];
    __shared__ uint64_t wc[WAVES];
    s = wave_sum(s);
    count = wave_sum(count);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        ws[wave] = s;
        wc[wave] = count;
    }
    __syncthreads();
    StatsRec rec{};
    if (threadIdx.x == 0) {
        double total = 0.0;
        uint64_t c = 0;
        for (int w = 0; w < WAVES; ++w) {
            total += ws[w];
            c += wc[w];
        }
        rec = write_record(out, total, c);
    }
    return rec;
}

// Row r of one gradient's analysis: elements [0, head) and the tail after
// the last whole 16-byte chunk are scalar (row 0); the body is walked in
// passes of STATS_BLOCK * STATS_UNROLL chunks, row r taking passes r,
// r + rows, r + 2 rows ...
template <int GDT>
__device__ __forceinline__ void analyze_row(const void *g, int64_t n, int32_t head, int64_t rows, int64_t r,
                                            StatsRec *out) {
    constexpr int EPC = GDT == G_F32 ? 4 : 8;  // elements per 16-byte chunk
    constexpr int64_t PASS = int64_t(STATS_BLOCK) * STATS_UNROLL;
    const int tid = threadIdx.x;
    const int64_t body = (n - head) / EPC;
    const void *gb = static_cast<const char *>(g) + int64_t(head) * (GDT == G_F32 ? 4 : 2);

    Acc a;
    a.s[0] = a.s[1] = a.s[2] = a.s[3] = 0.0;
    a.bad = 0;
    for (int64_t base = r * PASS; base < body; base += rows * PASS) {
        if (base + PASS <= body) {
#pragma unroll
            for (int u = 0; u < STATS_UNROLL; ++u) acc_chunk<GDT>(a, gb, base + u * STATS_BLOCK + tid);
        } else {
#pragma unroll
            for (int u = 0; u < STATS_UNROLL; ++u) {
                const int64_t k = base + u * STATS_BLOCK + tid;
                if (k < body) acc_chunk<GDT>(a, gb, k);
            }
        }
    }
    if (r == 0) {
        const int64_t tail = n - head - body * EPC;
        if (tid < head + tail) {
            const int64_t e = tid < head ? int64_t(tid) : head + body * EPC + (tid - head);
            acc_value(a, 0, load_one<GDT>(g, e));
        }
    }
    const double s = (a.s[0] + a.s[1]) + (a.s[2] + a.s[3]);
    block_finish<STATS_BLOCK>(s, a.bad, out);
}

// One gradient: workgroup b writes record b.
template <int GDT>
__global__ __launch_bounds__(STATS_BLOCK) void grad_analyze(const void *g, int64_t n, int32_t head,
                                                            int64_t rows, StatsRec *out) {
    analyze_row<GDT>(g, n, head, rows, blockIdx.x, out + blockIdx.x);
}

// Several gradients in one launch: workgroup b finds the gradient whose
// records include b and computes the same record a single-tensor launch
// would, so the reports are bit-identical.  coarse[j] is the gradient holding
// row j << STATS_COARSE_LOG2, so the search runs over [coarse[j],
// coarse[j + 1]] (usually one or two gradients) rather than the whole list:
// a list of a few hundred tensors otherwise spends about as long in the
// search's dependent loads as in streaming a 16 KiB row.
template <int GDT>
__global__ __launch_bounds__(STATS_BLOCK) void grad_analyze_table(const StatsSeg *__restrict__ segs,
                                                                  const int32_t *__restrict__ coarse,
                                                                  StatsRec *out) {
    const int64_t b = blockIdx.x;
    const int64_t j = b >> STATS_COARSE_LOG2;
    int32_t lo = coarse[j], hi = coarse[j + 1] + 1;  // segs[lo].row_begin <= b < segs[hi].row_begin
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (segs[mid].row_begin <= b) lo = mid; else hi = mid;
    }
    const StatsSeg sg = segs[lo];
    analyze_row<GDT>(sg.g, sg.n, sg.head, sg.rows, b - sg.row_begin, out + b);
}

// Workgroup b reduces records [b * per_block, min(nin, (b + 1) * per_block)).
__global__ __launch_bounds__(MERGE_BLOCK) void stats_merge(const StatsRec *in, int64_t nin,
                                                           int64_t per_block, StatsRec *out) {
    const int64_t begin = int64_t(blockIdx.x) * per_block;
    int64_t end = begin + per_block;
    if (end > nin) end = nin;
    double s = 0.0;
    uint64_t c = 0;
    for (int64_t r = begin + threadIdx.x; r < end; r += MERGE_BLOCK) {
        const StatsRec rec = in[r];
        s += __builtin_bit_cast(double, uint64_t(rec.w[0]) | (uint64_t(rec.w[1]) << 32));
        c += rec.w[2];
    }
    block_finish<MERGE_BLOCK>(s, c, out + blockIdx.x);
}

// Correctly rounded binary64 square root: the hardware estimate, then
// Tuckerman's test on its neighbours (y is the rounded root of x exactly
// when y * pred(y) < x <= y * succ(y); fma gives each product's difference
// from x with its exact sign).  The host's sqrt is correctly rounded, so
// both sides take the same decision from the same report.
__device__ __forceinline__ double sqrt_rn(double x) {
    if (!(x > 0.0)) return x;  // 0 (a sum of squares is never negative)
    double y = __builtin_sqrt(x);
    const uint64_t b = __builtin_bit_cast(uint64_t, y);
    const double below = __builtin_bit_cast(double, b - 1), above = __builtin_bit_cast(double, b + 1);
    if (__builtin_fma(y, below, -x) >= 0.0) y = below;
    else if (__builtin_fma(y, above, -x) < 0.0) y = above;
    return y;
}

// The fused step's decision from the merged report (TR-zh "在 ruda:0 上进行
// 原生 PyTorch 训练": a non-finite value skips the step, otherwise the global
// norm of the unscaled gradients is clipped), in the operation order of the
// host's radamw_decide and make_coefs: norm = sqrt(sumsq) / scale, clip =
// min(1, max_norm / (norm + 1e-6)), inv_scale = (float)(1 / (scale /
// clip)) before the sign of maximize is applied.  Every binary64 operation
// is correctly rounded on both sides.
__device__ Decision decide_on_device(double sumsq, uint32_t count, const DecideArgs &a) {
#pragma clang fp contract(off)
    Decision d;
    if (count > 0) {
        d.skip = 1;
        d.inv_scale = static_cast<float>(1.0 / a.gradient_scale);
        return d;
    }
    const double norm = sqrt_rn(sumsq) / a.gradient_scale;
    double clip = 1.0;
    if (a.max_grad_norm > 0.0) {
        const double q = a.max_grad_norm / (norm + 1e-6);
        clip = q < 1.0 ? q : 1.0;
    }
    const double eff = clip == 1.0 ? a.gradient_scale : a.gradient_scale / clip;
    d.skip = 0;
    d.inv_scale = static_cast<float>(1.0 / eff);
    return d;
}

// Final merge of a fused step (one workgroup): the report goes to `out` and
// the decision, taken from the report's own bits, to both dec pointers.
__global__ __launch_bounds__(MERGE_BLOCK) void stats_merge_decide(const StatsRec *in, int64_t nin, StatsRec *out,
                                                                  Decision *dec_dev, Decision *dec_host,
                                                                  DecideArgs a) {
    double s = 0.0;
    uint64_t c = 0;
    for (int64_t r = threadIdx.x; r < nin; r += MERGE_BLOCK) {
        const StatsRec rec = in[r];
        s += __builtin_bit_cast(double, uint64_t(rec.w[0]) | (uint64_t(rec.w[1]) << 32));
        c += rec.w[2];
    }
    const StatsRec rec = block_finish<MERGE_BLOCK>(s, c, out);
    if (threadIdx.x == 0) {
        // decide from exactly the words of the report
        const Decision d = decide_on_device(
            __builtin_bit_cast(double, uint64_t(rec.w[0]) | (uint64_t(rec.w[1]) << 32)), rec.w[2], a);
        *dec_dev = d;
        *dec_host = d;
        if (a.done) {
            // the host waits on this word: the report and the decision
            // reach host memory first
            __threadfence_system();
            *reinterpret_cast<volatile uint32_t *>(a.done) = a.seq;
        }
    }
}

// Static LDS of an analysis workgroup (block_finish's per-wave partials).
constexpr size_t ANALYZE_STATIC_LDS = (STATS_BLOCK / 64) * (sizeof(double) + sizeof(uint64_t));

// The FP32 analysis runs capped at STATS_F32_WG_PER_CU resident workgroups
// per CU; the 16-bit ones are uncapped.
inline size_t analyze_lds_reservation(int gdt) {
    return gdt == G_F32 ? lds_for_cap(STATS_F32_WG_PER_CU, ANALYZE_STATIC_LDS) : 0;
}

hipError_t launch_analyze(const void *g, int gdt, int64_t n, int32_t head, int64_t rows,
                          StatsRec *out, hipStream_t stream) {
    switch (gdt) {
    case G_F32:
        hipLaunchKernelGGL(grad_analyze<G_F32>, dim3(rows), dim3(STATS_BLOCK), analyze_lds_reservation(G_F32),
                           stream, g, n, head, rows, out);
        break;
    case G_F16:
        hipLaunchKernelGGL(grad_analyze<G_F16>, dim3(rows), dim3(STATS_BLOCK), 0, stream, g, n, head, rows, out);
        break;
    case G_BF16:
        hipLaunchKernelGGL(grad_analyze<G_BF16>, dim3(rows), dim3(STATS_BLOCK), 0, stream, g, n, head, rows, out);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_analyze_table(const StatsSeg *segs_dev, const int32_t *coarse_dev, int64_t total_rows,
                                int gdt, StatsRec *out, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(total_rows)), block(STATS_BLOCK);
    switch (gdt) {
    case G_F32:
        hipLaunchKernelGGL(grad_analyze_table<G_F32>, grid, block, analyze_lds_reservation(G_F32), stream, segs_dev,
                           coarse_dev, out);
        break;
    case G_F16: hipLaunchKernelGGL(grad_analyze_table<G_F16>, grid, block, 0, stream, segs_dev, coarse_dev, out); break;
    case G_BF16: hipLaunchKernelGGL(grad_analyze_table<G_BF16>, grid, block, 0, stream, segs_dev, coarse_dev, out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_merge(const StatsRec *in, int64_t nin, int64_t per_block, int64_t nblocks,
                        StatsRec *out, hipStream_t stream) {
    hipLaunchKernelGGL(stats_merge, dim3(nblocks), dim3(MERGE_BLOCK), 0, stream, in, nin, per_block, out);
    return hipGetLastError();
}

hipError_t launch_merge_decide(const StatsRec *in, int64_t nin, StatsRec *out, Decision *dec_dev,
                               Decision *dec_host, const DecideArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(stats_merge_decide, dim3(1), dim3(MERGE_BLOCK), 0, stream, in, nin, out, dec_dev, dec_host,
                       a);
    return hipGetLastError();
}

}  // namespace radamw
