// radamw_update.hip -- the fused AdamW / AMSGrad update kernels for gfx950.
//
// Page abbreviations: FA-ja = RUDA docs page "実験的なデバイス上の融合 AdamW /
// AMSGrad"; FA-zh = "实验性融合 AdamW / AMSGrad".
//
// One pass per element performs the whole update of FA-ja, section
// "この演算子を使用する理由": unscale (sign carries maximize), both moment
// EMAs, the optional AMSGrad running max (stored uncorrected), bias
// correction with epsilon outside the square root, decoupled weight decay
// and the parameter write.  The FIRST variants start the moments from zero
// inside the kernel and never read the moment arrays (FA-zh
// "增加的实际能力").
//
// The path is a pure stream (26-36 bytes and ~20 VALU ops per element), so
// the design is about HBM: every lane moves 16-byte chunks of each stream
// (global_load/store_dwordx4; 8-byte loads for 16-bit gradients), a wave
// covers 1 KiB contiguous per stream, all loads of a tile are issued before
// any arithmetic, and the data is touched exactly once, so loads and stores
// carry the nontemporal hint (measured: ~5% faster than default caching).
// Each workgroup is a single wave64 that handles one tile and exits, so the
// dispatcher keeps the whole chip busy with short, independent request
// streams; an LDS reservation at launch caps how many of them a CU holds at
// once, which HBM serves faster than a full CU.  No MFMA: there is no
// contraction here.
#include "radamw_math.h"

#include <hip/hip_ext.h>

namespace radamw {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

#ifndef RADAMW_NT_LOADS
#define RADAMW_NT_LOADS 1
#endif
#ifndef RADAMW_NT_STORES
#define RADAMW_NT_STORES 1
#endif
// 1: a workgroup reads the fused step's decision before it issues any tile
// load, so a skipped step moves no tile data; 0: after (the loads' latency
// then hides the decision's).
#ifndef RADAMW_DECISION_FIRST
#define RADAMW_DECISION_FIRST 0
#endif

template <typename T>
__device__ __forceinline__ T stream_load(const T *p) {
#if RADAMW_NT_LOADS
    return __builtin_nontemporal_load(gl(p));
#else
    return *gl(p);
#endif
}

template <typename T>
__device__ __forceinline__ void stream_store(T *p, T v) {
#if RADAMW_NT_STORES
    __builtin_nontemporal_store(v, gl(p));
#else
    *gl(p) = v;
#endif
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t upper_bits) {
    return __builtin_bit_cast(float, upper_bits);
}

// Four gradient values starting at element e (e % 4 == 0 relative to an
// aligned base), widened to FP32 exactly.
template <int GDT>
__device__ __forceinline__ f32x4 load_grad4(const void *g, int64_t e) {
    if constexpr (GDT == G_F32) {
        return stream_load(reinterpret_cast<const f32x4 *>(static_cast<const float *>(g) + e));
    } else if constexpr (GDT == G_F16) {
        f16x4 h = stream_load(reinterpret_cast<const f16x4 *>(static_cast<const _Float16 *>(g) + e));
        return __builtin_convertvector(h, f32x4);
    } else {
        u32x2 w = stream_load(reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(g) + e));
        f32x4 r;
        r.x = bf16_bits_to_float(w.x << 16);
        r.y = bf16_bits_to_float(w.x & 0xffff0000u);
        r.z = bf16_bits_to_float(w.y << 16);
        r.w = bf16_bits_to_float(w.y & 0xffff0000u);
        return r;
    }
}

template <int GDT>
__device__ __forceinline__ float load_grad1(const void *g, int64_t e) {
    if constexpr (GDT == G_F32) {
        return gl(static_cast<const float *>(g))[e];
    } else if constexpr (GDT == G_F16) {
        return static_cast<float>(gl(static_cast<const _Float16 *>(g))[e]);
    } else {
        return bf16_bits_to_float(uint32_t(gl(static_cast<const uint16_t *>(g))[e]) << 16);
    }
}

// The per-element update (FA-ja "この演算子を使用する理由"), built from the
// shared helpers of radamw_math.h.  FIRST starts the moments from zero
// without reading them.
template <bool AMS, bool FIRST>
__device__ __forceinline__ void adamw_element(float x, float &p, float &m, float &v, float &vmax,
                                              const Coefs &c) {
    const float g = unscale(x, c);
    m = first_moment(FIRST ? 0.0f : m, g, c);
    v = second_moment(FIRST ? 0.0f : v, g, c);
    float v_used = v;
    if constexpr (AMS) {
        v_used = fmaxf(FIRST ? 0.0f : vmax, v);
        vmax = v_used;
    }
    p = apply_step(p, step_delta(m, v_used, c), c);
}

template <int GDT, bool AMS, bool FIRST>
__device__ __forceinline__ void scalar_element(const SegDesc &s, int64_t e, const Coefs &c) {
    float x = load_grad1<GDT>(s.g, e);
    float p = gl(s.p_in)[e];
    float m = 0.0f, v = 0.0f, vmax = 0.0f;
    if constexpr (!FIRST) {
        m = gl(s.m_in)[e];
        v = gl(s.v_in)[e];
        if constexpr (AMS) vmax = gl(s.vmax_in)[e];
    }
    adamw_element<AMS, FIRST>(x, p, m, v, vmax, c);
    gl(s.p_out)[e] = p;
    if (s.model_kind == G_BF16) gl(static_cast<__bf16 *>(s.model))[e] = static_cast<__bf16>(p);
    else if (s.model_kind == G_F16) gl(static_cast<_Float16 *>(s.model))[e] = static_cast<_Float16>(p);
    gl(s.m_out)[e] = m;
    gl(s.v_out)[e] = v;
    if constexpr (AMS) gl(s.vmax_out)[e] = vmax;
}

// One tile of a mutually aligned segment: UPDATE_UNROLL 16-byte chunks per
// lane, loads first, then arithmetic and stores.  The last tile of the
// segment also handles the <= 3 head and <= 3 tail elements with scalar code.
// A fused step's decision, if any: `skip` and the clipped unscale factor,
// which takes the sign of the launch's own factor (maximize negates).  The
// load is uniform (one scalar load per workgroup, from L2).  Negation is
// exact and rounding to nearest even is symmetric, so the result has the
// bits of the host's (float)(sign / scale).
__device__ __forceinline__ bool read_decision(const Decision *dec, Coefs &c) {
    if (!dec) return false;
    const u32x2 d = *gl(reinterpret_cast<const u32x2 *>(dec));  // {skip, inv_scale bits}
    // the words go through scalars: this compiler lowers __builtin_bit_cast
    // of a vector element lvalue (d.y) to the vector's first element
    const uint32_t skip = d.x, inv_bits = d.y;
    c.inv_scale = __builtin_copysignf(__builtin_bit_cast(float, inv_bits), c.inv_scale);
    return skip != 0;
}

// Keeps the compiler from moving the tile's loads below, or the decision's
// load above, this point: the data loads go out first and the decision's
// latency hides behind them.
__device__ __forceinline__ void loads_issued() { asm volatile("" ::: "memory"); }

template <int GDT, bool AMS, bool FIRST>
__device__ __forceinline__ void vector_tile(const SegDesc &s, int64_t tile, const Coefs &c0, const Decision *dec) {
    constexpr int U = UPDATE_UNROLL;
    Coefs c = c0;
    const int tid = threadIdx.x;
    const int64_t head = s.head;
    const int64_t body = (s.n - head) >> 2;  // 16-byte chunks in the aligned body
    const int64_t base = tile * UPDATE_TILE_CHUNKS;

    const f32x4 *p_in = reinterpret_cast<const f32x4 *>(s.p_in + head);
    const f32x4 *m_in = reinterpret_cast<const f32x4 *>(s.m_in + head);
    const f32x4 *v_in = reinterpret_cast<const f32x4 *>(s.v_in + head);
    const f32x4 *x_in = reinterpret_cast<const f32x4 *>(s.vmax_in + head);
    f32x4 *p_out = reinterpret_cast<f32x4 *>(s.p_out + head);
    f32x4 *m_out = reinterpret_cast<f32x4 *>(s.m_out + head);
    f32x4 *v_out = reinterpret_cast<f32x4 *>(s.v_out + head);
    f32x4 *x_out = reinterpret_cast<f32x4 *>(s.vmax_out + head);

    // the model copy (round to nearest even: v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32)
    auto store_copy = [&](int64_t k, const f32x4 &P) {
        if (s.model_kind == G_BF16)
            stream_store(reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(s.model) + head) + k,
                         __builtin_convertvector(P, bf16x4));
        else if (s.model_kind == G_F16)
            stream_store(reinterpret_cast<f16x4 *>(static_cast<_Float16 *>(s.model) + head) + k,
                         __builtin_convertvector(P, f16x4));
    };

    auto chunk = [&](f32x4 G, f32x4 &P, f32x4 &M, f32x4 &V, f32x4 &X) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float p = P[j], m = M[j], v = V[j], x = X[j];
            adamw_element<AMS, FIRST>(G[j], p, m, v, x, c);
            P[j] = p; M[j] = m; V[j] = v; X[j] = x;
        }
    };

#if RADAMW_DECISION_FIRST
    if (read_decision(dec, c)) return;
#endif
    if (base + UPDATE_TILE_CHUNKS <= body) {
        f32x4 P[U], G[U], M[U], V[U], X[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = base + int64_t(u) * UPDATE_BLOCK + tid;
            G[u] = load_grad4<GDT>(s.g, head + 4 * k);
            P[u] = stream_load(p_in + k);
            if constexpr (!FIRST) {
                M[u] = stream_load(m_in + k);
                V[u] = stream_load(v_in + k);
                if constexpr (AMS) X[u] = stream_load(x_in + k);
            } else {
                M[u] = f32x4(0.0f); V[u] = f32x4(0.0f); X[u] = f32x4(0.0f);
            }
        }
#if !RADAMW_DECISION_FIRST
        loads_issued();
        if (read_decision(dec, c)) return;
#endif
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = base + int64_t(u) * UPDATE_BLOCK + tid;
            chunk(G[u], P[u], M[u], V[u], X[u]);
            stream_store(p_out + k, P[u]);
            store_copy(k, P[u]);
            stream_store(m_out + k, M[u]);
            stream_store(v_out + k, V[u]);
            if constexpr (AMS) stream_store(x_out + k, X[u]);
        }
    } else {
#if !RADAMW_DECISION_FIRST
        if (read_decision(dec, c)) return;
#endif
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = base + int64_t(u) * UPDATE_BLOCK + tid;
            if (k < body) {
                f32x4 G = load_grad4<GDT>(s.g, head + 4 * k);
                f32x4 P = stream_load(p_in + k);
                f32x4 M = f32x4(0.0f), V = f32x4(0.0f), X = f32x4(0.0f);
                if constexpr (!FIRST) {
                    M = stream_load(m_in + k);
                    V = stream_load(v_in + k);
                    if constexpr (AMS) X = stream_load(x_in + k);
                }
                chunk(G, P, M, V, X);
                stream_store(p_out + k, P);
                store_copy(k, P);
                stream_store(m_out + k, M);
                stream_store(v_out + k, V);
                if constexpr (AMS) stream_store(x_out + k, X);
            }
        }
    }

    const int64_t ntiles = segment_tiles(s.n, s.head);
    if (tile == ntiles - 1) {
        const int64_t tail = s.n - head - 4 * body;
        if (tid < head + tail) {
            const int64_t e = tid < head ? int64_t(tid) : head + 4 * body + (tid - head);
            scalar_element<GDT, AMS, FIRST>(s, e, c);
        }
    }
}

// One tile of a segment whose streams are not mutually 16-byte aligned
// (only possible for views at odd offsets): plain element-wise code.
template <int GDT, bool AMS, bool FIRST>
__device__ __forceinline__ void scalar_tile(const SegDesc &s, int64_t tile, const Coefs &c0, const Decision *dec) {
    Coefs c = c0;
    if (read_decision(dec, c)) return;
    const int64_t base = tile * UPDATE_TILE_ELEMS;
#pragma unroll 4
    for (int k = 0; k < 4 * UPDATE_UNROLL; ++k) {
        const int64_t e = base + int64_t(k) * UPDATE_BLOCK + threadIdx.x;
        if (e < s.n) scalar_element<GDT, AMS, FIRST>(s, e, c);
    }
}

template <int GDT, bool AMS, bool FIRST>
__device__ __forceinline__ void any_tile(const SegDesc &s, int64_t tile, const Coefs &c, const Decision *dec) {
    if (s.head >= 0)
        vector_tile<GDT, AMS, FIRST>(s, tile, c, dec);
    else
        scalar_tile<GDT, AMS, FIRST>(s, tile, c, dec);
}

// One tensor: the descriptor travels in the kernel arguments; workgroup t
// handles tile t (the host launches exactly one workgroup per tile).
template <int GDT, bool AMS, bool FIRST>
__global__ __launch_bounds__(UPDATE_BLOCK) void adamw_update_single(SegDesc s, Coefs c, const Decision *dec) {
    any_tile<GDT, AMS, FIRST>(s, blockIdx.x, c, dec);
}

// A list of tensors in one launch.  Descriptors, tile prefix sums and a
// coarse index live in device memory: coarse[j] is the segment holding tile
// j << TABLE_COARSE_LOG2, so a workgroup's segment lies in
// [coarse[j], coarse[j + 1]] and is found with one load and a short binary
// search (usually over one or two segments), instead of a search over the
// whole list before every 256-element tile.
template <int GDT, bool AMS, bool FIRST>
__global__ __launch_bounds__(UPDATE_BLOCK) void adamw_update_table(
    const SegDesc *__restrict__ segs, const int64_t *__restrict__ prefix,
    const int32_t *__restrict__ coarse, Coefs c, const Decision *dec) {
    const int64_t t = blockIdx.x;  // one workgroup per tile, grid == total_tiles
    const int64_t j = t >> TABLE_COARSE_LOG2;
    int32_t lo = coarse[j], hi = coarse[j + 1] + 1;  // prefix[lo] <= t < prefix[hi]
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (prefix[mid] <= t) lo = mid; else hi = mid;
    }
    const SegDesc seg = segs[lo];
    any_tile<GDT, AMS, FIRST>(seg, t - prefix[lo], c, dec);
}

// `lds` is the occupancy reservation (update_lds_reservation): dynamic LDS
// the kernels never touch, which caps the workgroups resident on a CU.
template <int GDT, bool AMS, bool FIRST>
static hipError_t launch_single_t(const SegDesc &seg, const Coefs &c, const Decision *dec, int grid,
                                  size_t lds, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
    hipExtLaunchKernelGGL((adamw_update_single<GDT, AMS, FIRST>), dim3(grid), dim3(UPDATE_BLOCK), lds,
                          st, start, stop, 0, seg, c, dec);
    return hipGetLastError();
}

template <int GDT, bool AMS, bool FIRST>
static hipError_t launch_table_t(const SegDesc *segs, const int64_t *prefix, const int32_t *coarse,
                                 const Coefs &c, const Decision *dec, int grid, size_t lds, hipStream_t st,
                                 hipEvent_t start, hipEvent_t stop) {
    hipExtLaunchKernelGGL((adamw_update_table<GDT, AMS, FIRST>), dim3(grid), dim3(UPDATE_BLOCK), lds,
                          st, start, stop, 0, segs, prefix, coarse, c, dec);
    return hipGetLastError();
}

#define RADAMW_DISPATCH(FN, ...)                                                      \
    switch (gdt * 4 + (amsgrad ? 2 : 0) + (first ? 1 : 0)) {                          \
    case 0: return FN<G_F32, false, false>(__VA_ARGS__);                              \
    case 1: return FN<G_F32, false, true>(__VA_ARGS__);                               \
    case 2: return FN<G_F32, true, false>(__VA_ARGS__);                               \
    case 3: return FN<G_F32, true, true>(__VA_ARGS__);                                \
    case 4: return FN<G_F16, false, false>(__VA_ARGS__);                              \
    case 5: return FN<G_F16, false, true>(__VA_ARGS__);                               \
    case 6: return FN<G_F16, true, false>(__VA_ARGS__);                               \
    case 7: return FN<G_F16, true, true>(__VA_ARGS__);                                \
    case 8: return FN<G_BF16, false, false>(__VA_ARGS__);                             \
    case 9: return FN<G_BF16, false, true>(__VA_ARGS__);                              \
    case 10: return FN<G_BF16, true, false>(__VA_ARGS__);                             \
    case 11: return FN<G_BF16, true, true>(__VA_ARGS__);                              \
    default: return hipErrorInvalidValue;                                             \
    }

hipError_t launch_update_single(const SegDesc &seg, const Coefs &c, const Decision *dec, int gdt,
                                bool amsgrad, bool first, int grid, hipStream_t stream, hipEvent_t start,
                                hipEvent_t stop) {
    const size_t lds = update_lds_reservation(gdt, amsgrad, first, seg.model_kind != 0);
    RADAMW_DISPATCH(launch_single_t, seg, c, dec, grid, lds, stream, start, stop)
}

hipError_t launch_update_table(const SegDesc *segs_dev, const int64_t *tile_prefix_dev,
                               const int32_t *coarse_dev, int32_t nseg, int64_t total_tiles,
                               const Coefs &c, const Decision *dec, int gdt, bool amsgrad, bool first,
                               bool copy, int grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    (void)nseg;
    (void)total_tiles;
    const size_t lds = update_lds_reservation(gdt, amsgrad, first, copy);
    RADAMW_DISPATCH(launch_table_t, segs_dev, tile_prefix_dev, coarse_dev, c, dec, grid, lds, stream, start, stop)
}

}  // namespace radamw
