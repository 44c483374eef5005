// radamw_staged.hip -- the staged (unfused) AdamW / AMSGrad baseline for
// gfx950, used only to measure what fusion saves.
//
// Page abbreviations: FA-ja = RUDA docs page "実験的なデバイス上の融合 AdamW /
// AMSGrad"; FA-zh = "实验性融合 AdamW / AMSGrad".
//
// FA-ja "割り当てとパフォーマンスのモデル" and FA-zh "优化点与边界" compare
// the fused kernel with a benchmark-only baseline that submits four kernels
// (five with AMSGrad), re-reads the gradient and goes through a delta
// buffer: 48 bytes per parameter instead of 28 (60 instead of 36).  The
// split taken here (a reading of that description):
//   K1  m     = b1 m + (1-b1) g                 read g, m      write m
//   K2  v     = b2 v + (1-b2) g g               read g, v      write v
//   K2' vmax  = max(vmax, v)          (AMSGrad) read vmax, v   write vmax
//   K3  delta = (lr/bc1) m / (sqrt(v_used/bc2) + eps)
//                                               read m, v_used write delta
//   K4  p     = p (1 - lr wd) - delta           read p, delta  write p
// = 12 (15) four-byte accesses per element.  Each kernel uses the fused
// kernel's geometry (one wave64 tile of 256 elements per workgroup,
// nontemporal dwordx4 streams) and exactly its per-element arithmetic, so the
// two paths give bit-identical results and differ only in traffic and
// launches.  All arrays must be 16-byte aligned; a tail of n % 4 elements is
// handled by lanes of the last workgroup.
#include "radamw_math.h"

namespace radamw {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int STAGED_BLOCK = 64;

template <typename T>
__device__ __forceinline__ T ld(const T *p) { return __builtin_nontemporal_load(gl(p)); }
template <typename T>
__device__ __forceinline__ void st(T *p, T v) { __builtin_nontemporal_store(v, gl(p)); }

template <int GDT>
__device__ __forceinline__ f32x4 grad4(const void *g, int64_t chunk) {
    if constexpr (GDT == G_F32) {
        return ld(reinterpret_cast<const f32x4 *>(g) + chunk);
    } else if constexpr (GDT == G_F16) {
        return __builtin_convertvector(ld(reinterpret_cast<const f16x4 *>(g) + chunk), f32x4);
    } else {
        const u32x2 w = ld(reinterpret_cast<const u32x2 *>(g) + chunk);
        f32x4 r;
        r.x = __builtin_bit_cast(float, w.x << 16);
        r.y = __builtin_bit_cast(float, w.x & 0xffff0000u);
        r.z = __builtin_bit_cast(float, w.y << 16);
        r.w = __builtin_bit_cast(float, w.y & 0xffff0000u);
        return r;
    }
}

template <int GDT>
__device__ __forceinline__ float grad1(const void *g, int64_t e) {
    if constexpr (GDT == G_F32) return gl(static_cast<const float *>(g))[e];
    else if constexpr (GDT == G_F16) return static_cast<float>(gl(static_cast<const _Float16 *>(g))[e]);
    else return __builtin_bit_cast(float, uint32_t(gl(static_cast<const uint16_t *>(g))[e]) << 16);
}

// Element index range of this lane: one 4-element chunk of the body, or one
// element of the n % 4 tail (lanes of the last workgroup past the body).
struct Lane {
    int64_t chunk;  // >= 0: vector chunk index
    int64_t tail;   // >= 0: scalar element index
};

__device__ __forceinline__ Lane lane_of(int64_t n) {
    const int64_t body = n >> 2;
    const int64_t k = int64_t(blockIdx.x) * STAGED_BLOCK + threadIdx.x;
    if (k < body) return {k, -1};
    const int64_t e = 4 * body + (k - body);
    return {-1, e < n ? e : -1};
}

// K1: first moment.
template <int GDT, bool FIRST>
__global__ __launch_bounds__(STAGED_BLOCK) void staged_m(const void *g, float *m, int64_t n, Coefs c) {
    const Lane l = lane_of(n);
    if (l.chunk >= 0) {
        const f32x4 x = grad4<GDT>(g, l.chunk);
        const f32x4 m0 = FIRST ? f32x4(0.0f) : ld(reinterpret_cast<const f32x4 *>(m) + l.chunk);
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = first_moment(m0[j], unscale(x[j], c), c);
        st(reinterpret_cast<f32x4 *>(m) + l.chunk, r);
    } else if (l.tail >= 0) {
        const float m0 = FIRST ? 0.0f : gl(m)[l.tail];
        gl(m)[l.tail] = first_moment(m0, unscale(grad1<GDT>(g, l.tail), c), c);
    }
}

// K2: second moment.
template <int GDT, bool FIRST>
__global__ __launch_bounds__(STAGED_BLOCK) void staged_v(const void *g, float *v, int64_t n, Coefs c) {
    const Lane l = lane_of(n);
    if (l.chunk >= 0) {
        const f32x4 x = grad4<GDT>(g, l.chunk);
        const f32x4 v0 = FIRST ? f32x4(0.0f) : ld(reinterpret_cast<const f32x4 *>(v) + l.chunk);
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = second_moment(v0[j], unscale(x[j], c), c);
        st(reinterpret_cast<f32x4 *>(v) + l.chunk, r);
    } else if (l.tail >= 0) {
        const float v0 = FIRST ? 0.0f : gl(v)[l.tail];
        gl(v)[l.tail] = second_moment(v0, unscale(grad1<GDT>(g, l.tail), c), c);
    }
}

// K2': AMSGrad running max (uncorrected).
template <bool FIRST>
__global__ __launch_bounds__(STAGED_BLOCK) void staged_vmax(const float *v, float *vmax, int64_t n) {
    const Lane l = lane_of(n);
    if (l.chunk >= 0) {
        const f32x4 a = ld(reinterpret_cast<const f32x4 *>(v) + l.chunk);
        const f32x4 b = FIRST ? f32x4(0.0f) : ld(reinterpret_cast<const f32x4 *>(vmax) + l.chunk);
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = fmaxf(b[j], a[j]);
        st(reinterpret_cast<f32x4 *>(vmax) + l.chunk, r);
    } else if (l.tail >= 0) {
        const float b = FIRST ? 0.0f : gl(vmax)[l.tail];
        gl(vmax)[l.tail] = fmaxf(b, gl(v)[l.tail]);
    }
}

// K3: the bias-corrected step into the delta buffer.
__global__ __launch_bounds__(STAGED_BLOCK) void staged_delta(const float *m, const float *vu, float *delta,
                                                             int64_t n, Coefs c) {
    const Lane l = lane_of(n);
    if (l.chunk >= 0) {
        const f32x4 a = ld(reinterpret_cast<const f32x4 *>(m) + l.chunk);
        const f32x4 b = ld(reinterpret_cast<const f32x4 *>(vu) + l.chunk);
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = step_delta(a[j], b[j], c);
        st(reinterpret_cast<f32x4 *>(delta) + l.chunk, r);
    } else if (l.tail >= 0) {
        gl(delta)[l.tail] = step_delta(gl(m)[l.tail], gl(vu)[l.tail], c);
    }
}

// K4: decoupled decay and the parameter write.
__global__ __launch_bounds__(STAGED_BLOCK) void staged_param(float *p, const float *delta, int64_t n, Coefs c) {
    const Lane l = lane_of(n);
    if (l.chunk >= 0) {
        const f32x4 a = ld(reinterpret_cast<const f32x4 *>(p) + l.chunk);
        const f32x4 d = ld(reinterpret_cast<const f32x4 *>(delta) + l.chunk);
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = apply_step(a[j], d[j], c);
        st(reinterpret_cast<f32x4 *>(p) + l.chunk, r);
    } else if (l.tail >= 0) {
        gl(p)[l.tail] = apply_step(gl(p)[l.tail], gl(delta)[l.tail], c);
    }
}

template <int GDT, bool FIRST>
static hipError_t staged_all(float *p, const void *g, float *m, float *v, float *vmax, float *delta,
                             int64_t n, const Coefs &c, hipStream_t s, int *launched) {
    const int64_t lanes = (n >> 2) + (n & 3);
    const dim3 grid(static_cast<unsigned>((lanes + STAGED_BLOCK - 1) / STAGED_BLOCK)), block(STAGED_BLOCK);
    // the fused kernels' occupancy rule, from each kernel's own streams
    constexpr int64_t gb = GDT == G_F32 ? 4 : 2;
    const size_t lds_moment = stream_lds_reservation(gb + (FIRST ? 4 : 8));  // g, [m or v], m or v
    const size_t lds_vmax = stream_lds_reservation(FIRST ? 8 : 12);          // v, [vmax], vmax
    const size_t lds_rest = stream_lds_reservation(12);                      // two reads, one write
    hipError_t e;
    *launched = 0;
    hipLaunchKernelGGL((staged_m<GDT, FIRST>), grid, block, lds_moment, s, g, m, n, c);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    ++*launched;
    hipLaunchKernelGGL((staged_v<GDT, FIRST>), grid, block, lds_moment, s, g, v, n, c);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    ++*launched;
    const float *vu = v;
    if (vmax) {
        hipLaunchKernelGGL((staged_vmax<FIRST>), grid, block, lds_vmax, s, v, vmax, n);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        ++*launched;
        vu = vmax;
    }
    hipLaunchKernelGGL(staged_delta, grid, block, lds_rest, s, m, vu, delta, n, c);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    ++*launched;
    hipLaunchKernelGGL(staged_param, grid, block, lds_rest, s, p, delta, n, c);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    ++*launched;
    return hipSuccess;
}

hipError_t launch_staged(float *p, const void *g, int gdt, float *m, float *v, float *vmax, float *delta,
                         int64_t n, bool first, const Coefs &c, hipStream_t stream, int *launched) {
    switch (gdt * 2 + (first ? 1 : 0)) {
    case 0: return staged_all<G_F32, false>(p, g, m, v, vmax, delta, n, c, stream, launched);
    case 1: return staged_all<G_F32, true>(p, g, m, v, vmax, delta, n, c, stream, launched);
    case 2: return staged_all<G_F16, false>(p, g, m, v, vmax, delta, n, c, stream, launched);
    case 3: return staged_all<G_F16, true>(p, g, m, v, vmax, delta, n, c, stream, launched);
    case 4: return staged_all<G_BF16, false>(p, g, m, v, vmax, delta, n, c, stream, launched);
    case 5: return staged_all<G_BF16, true>(p, g, m, v, vmax, delta, n, c, stream, launched);
    default: *launched = 0; return hipErrorInvalidValue;
    }
}

}  // namespace radamw
