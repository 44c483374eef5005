// radamw_api.cpp -- the C ABI of libradamw.so: validation, host-side
// coefficients, launch geometry, segment tables and the statistics plan.
//
// Page abbreviations: FA-ja = RUDA docs page "実験的なデバイス上の融合 AdamW /
// AMSGrad"; FA-zh = "实验性融合 AdamW / AMSGrad"; TR-zh = "训练与状态保存".
//
// Every entry point validates all of its arguments before it launches or
// writes anything (FA-ja "低レベルの使用"), so a failed call has no effect.
#include "radamw.h"
#include "radamw_internal.h"

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstring>
#include <limits>
#include <map>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

using namespace radamw;

namespace {

std::atomic<uint64_t> g_launches{0};
thread_local int g_last_hip = 0;

// Measurement hook (radamw_time_next_update): events for the next call on
// this thread that launches an update.
struct UpdateTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
thread_local UpdateTiming g_timing;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return RADAMW_OK;
    g_last_hip = static_cast<int>(e);
    return RADAMW_ERR_HIP;
}

// ------------------------------------------------------------ device info --

constexpr int MAX_DEVICES = 64;

struct DeviceCache {
    std::mutex mu;
    // segment-table staging ring (see launch_table)
    static constexpr int RING = 8;
    struct Slot {
        void *host = nullptr;
        void *dev = nullptr;
        size_t cap = 0;
        hipEvent_t done = nullptr;
        bool pending = false;
    } slots[RING];
    int next = 0;
    // pinned 12-byte staging for report read-back
    radamw_stats *pinned_report = nullptr;
    // host memory mapped for the device: the fused step's final merge writes
    // its report (offset 0), its decision (offset 16) and then the call's
    // sequence number (offset 32) here directly, so the read-back is the host
    // watching that word (report_mu)
    std::mutex report_mu;
    radamw_stats *mapped_report_host = nullptr;
    radamw_stats *mapped_report_dev = nullptr;
    Decision *mapped_decision_host = nullptr;
    Decision *mapped_decision_dev = nullptr;
    volatile uint32_t *mapped_done_host = nullptr;
    uint32_t *mapped_done_dev = nullptr;
    uint32_t done_seq = 0;
    // one merged record per list of a multi-list fused step (report_mu)
    StatsRec *group_rec = nullptr;
    int64_t group_cap = 0;
    // a second stream for the update launches of a multi-tensor step
    // (aux_mu): every other launch goes to it, so that one tensor's drain
    // overlaps the next tensor's ramp; fork / join order it after the
    // caller's earlier work and the caller's later work after it
    std::mutex aux_mu;
    hipStream_t aux = nullptr;
    hipEvent_t fork = nullptr;
    hipEvent_t join = nullptr;
    // radamw_fused_step_multi_noalloc: the device address of this device's
    // copy of `scratch` (found once), and the lock that serialises the
    // calls sharing it
    std::mutex noalloc_mu;
    char *noalloc_scratch = nullptr;
};

DeviceCache g_devices[MAX_DEVICES];

// ------------------------------------------- allocation-free fused step --
//
// radamw_fused_step_multi_noalloc keeps what radamw_fused_step_multi puts in
// the caller's workspace -- the statistics rows, the merge scratch and the
// decision slot, laid out exactly as in a workspace -- in this file-scope
// device array, followed by the 12-byte report and a second copy of the
// decision, which the host reads back together.  It is sized for the largest
// single-segment step: a tensor writes at most STATS_ROWS_CAP rows, whose
// fan-in-1024 merge needs ceil(STATS_ROWS_CAP / 1024) intermediate records.
constexpr int64_t noalloc_merge_records(int64_t rows) {
    return rows > MERGE_FAN_IN ? (rows + MERGE_FAN_IN - 1) / MERGE_FAN_IN + noalloc_merge_records(
                                     (rows + MERGE_FAN_IN - 1) / MERGE_FAN_IN) : 0;
}
constexpr int64_t NOALLOC_WORKSPACE_BYTES = STATS_ROWS_CAP * 12 + noalloc_merge_records(STATS_ROWS_CAP) * 12 + 12;
constexpr int64_t NOALLOC_REPORT_OFF = (NOALLOC_WORKSPACE_BYTES + 15) / 16 * 16;  // report: 12 B
constexpr int64_t NOALLOC_DEC_COPY_OFF = NOALLOC_REPORT_OFF + 16;                   // decision copy: 8 B
constexpr int64_t NOALLOC_SCRATCH_BYTES = (NOALLOC_DEC_COPY_OFF + 8 + 255) / 256 * 256;
static_assert(NOALLOC_SCRATCH_BYTES <= 128 * 1024, "the allocation-free step's scratch stays modest");

static __device__ __align__(256) uint64_t scratch[NOALLOC_SCRATCH_BYTES / 8];

// Temporarily make `dev` the calling thread's current device.
struct DeviceScope {
    int prev = -1;
    explicit DeviceScope(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) (void)hipSetDevice(dev);
    }
    ~DeviceScope() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// The device of `stream`; a stream being captured into a graph is refused
// (a replay would repeat one step's host-formed coefficients, and a fused
// step waits for its own kernels, which a capture never runs).
int stream_device(hipStream_t stream, int *dev) {
    hipDevice_t d = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &d) : hipGetDevice(&d);
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (e == hipSuccess) e = hipStreamIsCapturing(stream, &capture);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        g_last_hip = static_cast<int>(e);
        return RADAMW_ERR_INVALID;
    }
    if (capture != hipStreamCaptureStatusNone) return RADAMW_ERR_INVALID;
    if (d < 0 || d >= MAX_DEVICES) return RADAMW_ERR_INVALID;
    *dev = static_cast<int>(d);
    return RADAMW_OK;
}

// ------------------------------------------------------------- validation --

bool is_finite(double x) { return std::isfinite(x); }

int check_options(const radamw_options *o) {
    if (!o) return RADAMW_ERR_INVALID;
    if (!is_finite(o->lr) || o->lr < 0.0) return RADAMW_ERR_INVALID;
    if (!is_finite(o->eps) || o->eps < 0.0) return RADAMW_ERR_INVALID;
    if (!is_finite(o->weight_decay) || o->weight_decay < 0.0) return RADAMW_ERR_INVALID;
    if (!(o->beta1 >= 0.0 && o->beta1 < 1.0)) return RADAMW_ERR_INVALID;
    if (!(o->beta2 >= 0.0 && o->beta2 < 1.0)) return RADAMW_ERR_INVALID;
    if ((o->amsgrad != 0 && o->amsgrad != 1) || (o->maximize != 0 && o->maximize != 1))
        return RADAMW_ERR_INVALID;
    return RADAMW_OK;
}

int check_scale(double gradient_scale) {
    return (is_finite(gradient_scale) && gradient_scale > 0.0) ? RADAMW_OK : RADAMW_ERR_INVALID;
}

int check_control(const radamw_control *c) {
    if (!c) return RADAMW_ERR_INVALID;
    if (c->skip_update != 0 && c->skip_update != 1) return RADAMW_ERR_INVALID;
    return check_scale(c->gradient_scale);
}

bool valid_dtype(int gdt) { return gdt == RADAMW_F32 || gdt == RADAMW_F16 || gdt == RADAMW_BF16; }

size_t grad_bytes(int gdt) { return gdt == RADAMW_F32 ? 4 : 2; }

// Flattened-bucket placement (radamw_bucket_layout): stream k of a bucket
// starts at k * pitch in one allocation, pitch = its largest stream rounded
// up to 2 MiB plus 12 KiB.  Measured on MI355X: streams whose starts differ
// by exact multiples of large powers of two (1 GiB apart, or separately
// allocated 2 MiB-aligned buffers) update 3-6% slower than streams whose
// starts are further shifted by 4-20 KiB or 1 MiB, for streams of up to
// about 1 GiB; 12 KiB was best or within noise of the best for every
// variant swept.  Streams of 5-27 GB came within +-2% of separate
// allocations either way.
constexpr int64_t BUCKET_PITCH_ALIGN = int64_t(2) << 20;
constexpr int64_t BUCKET_STREAM_SHIFT = int64_t(12) << 10;

// Element counts above this are rejected (RADAMW_ERR_RANGE) before any byte
// size is formed, so n * element size cannot overflow; any tensor that fits
// in device memory is far below it.
constexpr int64_t MAX_ELEMENTS = int64_t(1) << 48;

// Pointer validation for one call.  A pointer must be device (or managed)
// memory of the stream's device, aligned to its element size, and the bytes
// the call touches must lie inside the allocation that holds it.  Each
// allocation is queried once per call (hipPointerGetAttributes and
// hipMemGetAddressRange); later pointers into an allocation already seen are
// checked against its cached extent, so a list of many tensors carved from
// a few allocations costs a few HIP queries, not one per pointer.
class PtrChecker {
  public:
    explicit PtrChecker(int dev) : dev_(dev) {}

    int check(const void *p, size_t align, int64_t bytes) {
        if (!p) return RADAMW_ERR_INVALID;
        const uintptr_t a = reinterpret_cast<uintptr_t>(p);
        if (a % align != 0) return RADAMW_ERR_ALIGN;
        const uintptr_t end = a + static_cast<uintptr_t>(bytes > 0 ? bytes : 0);
        auto it = known_.upper_bound(a);
        if (it != known_.begin()) {
            --it;
            if (a >= it->first && a < it->second) return end <= it->second ? RADAMW_OK : RADAMW_ERR_INVALID;
        }
        hipPointerAttribute_t attr;
        std::memset(&attr, 0, sizeof attr);
        hipError_t e = hipPointerGetAttributes(&attr, p);
        if (e != hipSuccess) {
            (void)hipGetLastError();  // leave no sticky error behind for the caller
            return RADAMW_ERR_INVALID;
        }
        if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return RADAMW_ERR_INVALID;
        if (attr.device != dev_) return RADAMW_ERR_INVALID;
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        e = hipMemGetAddressRange(&base, &size, const_cast<void *>(p));
        if (e != hipSuccess || !base || size == 0) {
            (void)hipGetLastError();
            return RADAMW_OK;  // extent unknown (e.g. managed memory): type and device checked
        }
        const uintptr_t lo = reinterpret_cast<uintptr_t>(base), hi = lo + size;
        if (a < lo || a >= hi) return RADAMW_OK;
        known_[lo] = hi;
        return end <= hi ? RADAMW_OK : RADAMW_ERR_INVALID;
    }

  private:
    int dev_;
    std::map<uintptr_t, uintptr_t> known_;  // allocation base -> end
};

// Byte ranges touched by one call.  Written ranges may overlap nothing;
// read-only ranges may overlap each other.
struct Range {
    uintptr_t lo, hi;
    bool written;
};

void add_range(std::vector<Range> &v, const void *p, int64_t bytes, bool written) {
    if (p && bytes > 0) {
        uintptr_t lo = reinterpret_cast<uintptr_t>(p);
        v.push_back({lo, lo + static_cast<uintptr_t>(bytes), written});
    }
}

// Sweep in start order: a written range must start after every earlier
// range ended; a read range must start after every earlier written range.
int check_alias(std::vector<Range> &v) {
    std::sort(v.begin(), v.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
    uintptr_t end_any = 0, end_written = 0;
    for (const Range &r : v) {
        if (r.written ? r.lo < end_any : r.lo < end_written) return RADAMW_ERR_ALIAS;
        end_any = std::max(end_any, r.hi);
        if (r.written) end_written = std::max(end_written, r.hi);
    }
    return RADAMW_OK;
}

// ----------------------------------------------------------- coefficients --

// beta^t in FP64 by binary exponentiation (an integer power, FA-ja
// "この演算子を使用する理由").
double int_pow(double base, uint64_t e) {
    double r = 1.0;
    while (e) {
        if (e & 1) r *= base;
        base *= base;
        e >>= 1;
    }
    return r;
}

// FP64 formation and FP32 cast of every per-call constant, once per call.
Coefs make_coefs(const radamw_options &o, uint64_t t, double gradient_scale) {
    const double bc1 = 1.0 - int_pow(o.beta1, t);
    const double bc2 = 1.0 - int_pow(o.beta2, t);
    Coefs c;
    c.beta1 = static_cast<float>(o.beta1);
    c.one_minus_beta1 = static_cast<float>(1.0 - o.beta1);
    c.beta2 = static_cast<float>(o.beta2);
    c.one_minus_beta2 = static_cast<float>(1.0 - o.beta2);
    c.inv_scale = static_cast<float>((o.maximize ? -1.0 : 1.0) / gradient_scale);
    c.decay = static_cast<float>(1.0 - o.lr * o.weight_decay);
    c.step_size = static_cast<float>(o.lr / bc1);
    c.inv_bc2 = static_cast<float>(1.0 / bc2);
    c.eps = static_cast<float>(o.eps);
    return c;
}

// ----------------------------------------------------------- segment geometry

bool same_phase(const void *q, int phase) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(q);
    return (a & 3) == 0 && static_cast<int>((a >> 2) & 3) == phase;
}

// Leading scalar elements so that all streams are 16-byte aligned after
// them, or -1 when the streams' alignments differ.
int32_t segment_head(const SegDesc &s, int gdt, bool amsgrad, bool first) {
    const int phase = static_cast<int>((reinterpret_cast<uintptr_t>(s.p_in) >> 2) & 3);
    bool ok = same_phase(s.p_out, phase) && same_phase(s.m_out, phase) && same_phase(s.v_out, phase);
    if (amsgrad) ok = ok && same_phase(s.vmax_out, phase);
    if (!first) {
        ok = ok && same_phase(s.m_in, phase) && same_phase(s.v_in, phase);
        if (amsgrad) ok = ok && same_phase(s.vmax_in, phase);
    }
    const uintptr_t ga = reinterpret_cast<uintptr_t>(s.g);
    const int gphase = gdt == RADAMW_F32 ? static_cast<int>((ga >> 2) & 3) : static_cast<int>((ga >> 1) & 3);
    ok = ok && gphase == phase;
    if (s.model_kind) {
        const uintptr_t ma = reinterpret_cast<uintptr_t>(s.model);
        ok = ok && (ma & 1) == 0 && static_cast<int>((ma >> 1) & 3) == phase;
    }
    if (!ok) return -1;
    int64_t head = (4 - phase) & 3;
    if (head > s.n) head = s.n;
    return static_cast<int32_t>(head);
}

// One workgroup per tile; callers have checked tiles <= UPDATE_MAX_GRID.
int update_grid(int64_t tiles) { return static_cast<int>(tiles); }

// Validate one tensor's pointers for an update; appends its byte ranges.
// For an out-of-place call the inputs are read-only ranges and the outputs
// written ones; in place, the state and parameter ranges are written.
int check_update_tensor(const SegDesc &s, int gdt, bool amsgrad, bool first, bool inplace,
                        PtrChecker &pc, std::vector<Range> &ranges) {
    const int64_t fb = s.n * 4, gb = s.n * static_cast<int64_t>(grad_bytes(gdt));
    int rc;
    if (!inplace && (rc = pc.check(s.p_in, 4, fb))) return rc;
    if ((rc = pc.check(s.g, grad_bytes(gdt), gb))) return rc;
    if ((rc = pc.check(s.p_out, 4, fb))) return rc;
    if ((rc = pc.check(s.m_out, 4, fb))) return rc;
    if ((rc = pc.check(s.v_out, 4, fb))) return rc;
    if (amsgrad && (rc = pc.check(s.vmax_out, 4, fb))) return rc;
    if (!first && !inplace) {
        if ((rc = pc.check(s.m_in, 4, fb))) return rc;
        if ((rc = pc.check(s.v_in, 4, fb))) return rc;
        if (amsgrad && (rc = pc.check(s.vmax_in, 4, fb))) return rc;
    }
    add_range(ranges, s.g, gb, false);
    if (inplace) {
        add_range(ranges, s.p_out, fb, true);
        add_range(ranges, s.m_out, fb, true);
        add_range(ranges, s.v_out, fb, true);
        if (amsgrad) add_range(ranges, s.vmax_out, fb, true);
    } else {
        add_range(ranges, s.p_in, fb, false);
        if (!first) {
            add_range(ranges, s.m_in, fb, false);
            add_range(ranges, s.v_in, fb, false);
            if (amsgrad) add_range(ranges, s.vmax_in, fb, false);
        }
        add_range(ranges, s.p_out, fb, true);
        add_range(ranges, s.m_out, fb, true);
        add_range(ranges, s.v_out, fb, true);
        if (amsgrad) add_range(ranges, s.vmax_out, fb, true);
    }
    return RADAMW_OK;
}

int launch_single(SegDesc s, int gdt, bool amsgrad, bool first, const Coefs &c, const Decision *dec, int dev,
                  hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
    (void)dev;
    s.head = segment_head(s, gdt, amsgrad, first);
    s.tile_begin = 0;
    const int64_t tiles = segment_tiles(s.n, s.head);
    if (tiles > UPDATE_MAX_GRID) return RADAMW_ERR_RANGE;
    const int grid = update_grid(tiles);
    int rc = hip_status(launch_update_single(s, c, dec, gdt, amsgrad, first, grid, stream, ev_start, ev_stop));
    if (rc == RADAMW_OK) g_launches.fetch_add(1, std::memory_order_relaxed);
    return rc;
}

// Per-launch tables for the multi-tensor kernels: `fill` writes `bytes` of
// table into pinned host memory, which is copied to a device slot on the
// caller's stream; `launch` receives the slot's device address.  A slot is
// recycled once an event shows that the kernel reading it has finished.
template <typename Fill, typename Launch>
int staged_launch(int dev, hipStream_t stream, size_t bytes, Fill fill, Launch launch) {
    DeviceCache &dc = g_devices[dev];
    std::lock_guard<std::mutex> lock(dc.mu);
    DeviceCache::Slot &slot = dc.slots[dc.next];
    dc.next = (dc.next + 1) % DeviceCache::RING;
    if (slot.pending) {
        hipError_t e = hipEventSynchronize(slot.done);
        if (e != hipSuccess) return hip_status(e);
        slot.pending = false;
    }
    if (!slot.done) {
        hipError_t e = hipEventCreateWithFlags(&slot.done, hipEventDisableTiming);
        if (e != hipSuccess) return hip_status(e);
    }
    if (slot.cap < bytes) {
        if (slot.host) (void)hipHostFree(slot.host);
        if (slot.dev) (void)hipFree(slot.dev);
        slot.host = slot.dev = nullptr;
        slot.cap = 0;
        size_t cap = std::max<size_t>(bytes, 64 * 1024);
        hipError_t e = hipHostMalloc(&slot.host, cap, hipHostMallocDefault);
        if (e != hipSuccess) return hip_status(e);
        e = hipMalloc(&slot.dev, cap);
        if (e != hipSuccess) {
            (void)hipHostFree(slot.host);
            slot.host = nullptr;
            return hip_status(e);
        }
        slot.cap = cap;
    }
    fill(static_cast<char *>(slot.host));
    hipError_t e = hipMemcpyAsync(slot.dev, slot.host, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_status(e);
    e = launch(static_cast<const char *>(slot.dev));
    if (e != hipSuccess) return hip_status(e);
    g_launches.fetch_add(1, std::memory_order_relaxed);
    e = hipEventRecord(slot.done, stream);
    if (e != hipSuccess) return hip_status(e);
    slot.pending = true;
    return RADAMW_OK;
}

// The device table of a multi-tensor update launch: descriptors, tile
// prefix sums and a coarse index, packed into one byte image.
struct UpdateTable {
    std::vector<char> bytes;
    size_t prefix_off = 0, coarse_off = 0;
    int32_t nseg = 0;
    int64_t tiles = 0;
    bool copy = false;  // some segment writes a model copy
};

int build_update_table(std::vector<SegDesc> &segs, int gdt, bool amsgrad, bool first, UpdateTable *t) {
    const int32_t nseg = static_cast<int32_t>(segs.size());
    std::vector<int64_t> prefix(nseg + 1);
    int64_t tiles = 0;
    for (int32_t i = 0; i < nseg; ++i) {
        segs[i].head = segment_head(segs[i], gdt, amsgrad, first);
        segs[i].tile_begin = tiles;
        prefix[i] = tiles;
        tiles += segment_tiles(segs[i].n, segs[i].head);
    }
    prefix[nseg] = tiles;
    if (tiles > UPDATE_MAX_GRID) return RADAMW_ERR_RANGE;
    // coarse[j] = the (non-empty) segment holding tile j << TABLE_COARSE_LOG2;
    // the last entry closes the range with the last segment.
    const int64_t ncoarse = ((tiles - 1) >> TABLE_COARSE_LOG2) + 1;
    std::vector<int32_t> coarse(ncoarse + 1);
    {
        int32_t s = 0;
        for (int64_t j = 0; j < ncoarse; ++j) {
            const int64_t tile = j << TABLE_COARSE_LOG2;
            while (prefix[s + 1] <= tile) ++s;
            coarse[j] = s;
        }
        coarse[ncoarse] = nseg - 1;
    }
    const size_t desc_bytes = sizeof(SegDesc) * nseg;
    const size_t prefix_bytes = sizeof(int64_t) * (nseg + 1);
    const size_t coarse_bytes = sizeof(int32_t) * (ncoarse + 1);
    t->bytes.resize(desc_bytes + prefix_bytes + coarse_bytes);
    t->prefix_off = desc_bytes;
    t->coarse_off = desc_bytes + prefix_bytes;
    std::memcpy(t->bytes.data(), segs.data(), desc_bytes);
    std::memcpy(t->bytes.data() + t->prefix_off, prefix.data(), prefix_bytes);
    std::memcpy(t->bytes.data() + t->coarse_off, coarse.data(), coarse_bytes);
    t->nseg = nseg;
    t->tiles = tiles;
    t->copy = std::any_of(segs.begin(), segs.end(), [](const SegDesc &d) { return d.model_kind != 0; });
    return RADAMW_OK;
}

// Launch an update over a table already in device memory at `base`.
hipError_t launch_table_at(const UpdateTable &t, const char *base, int gdt, bool amsgrad, bool first,
                           const Coefs &c, const Decision *dec, hipStream_t stream, hipEvent_t ev_start,
                           hipEvent_t ev_stop) {
    return launch_update_table(reinterpret_cast<const SegDesc *>(base),
                               reinterpret_cast<const int64_t *>(base + t.prefix_off),
                               reinterpret_cast<const int32_t *>(base + t.coarse_off), t.nseg, t.tiles, c, dec,
                               gdt, amsgrad, first, t.copy, update_grid(t.tiles), stream, ev_start, ev_stop);
}

// Several tensors in one launch, the table going through a staged slot
// (staged_launch).
int launch_table(std::vector<SegDesc> &segs, int gdt, bool amsgrad, bool first, const Coefs &c,
                 const Decision *dec, int dev, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
    UpdateTable t;
    int rc = build_update_table(segs, gdt, amsgrad, first, &t);
    if (rc) return rc;
    return staged_launch(
        dev, stream, t.bytes.size(), [&](char *host) { std::memcpy(host, t.bytes.data(), t.bytes.size()); },
        [&](const char *dev_base) {
            return launch_table_at(t, dev_base, gdt, amsgrad, first, c, dec, stream, ev_start, ev_stop);
        });
}

// In-place descriptors of the non-empty segments of a list; models
// (optional) holds a 16-bit model copy per segment (entries may be null), of
// dtype model_dtype.
std::vector<SegDesc> inplace_descs(const radamw_segment *segs, int32_t nseg, void *const *models,
                                   int model_dtype) {
    std::vector<SegDesc> active;
    active.reserve(static_cast<size_t>(nseg));
    for (int32_t i = 0; i < nseg; ++i) {
        const radamw_segment &s = segs[i];
        if (s.n == 0) continue;
        SegDesc d{};
        d.p_in = d.p_out = s.param;
        d.g = s.grad;
        d.m_in = d.m_out = s.exp_avg;
        d.v_in = d.v_out = s.exp_avg_sq;
        d.vmax_in = d.vmax_out = s.max_exp_avg_sq;
        d.n = s.n;
        if (models && models[i]) {
            d.model = models[i];
            d.model_kind = model_dtype == RADAMW_BF16 ? G_BF16 : G_F16;
        }
        active.push_back(d);
    }
    return active;
}

// Consecutive tensors of a list that continue one another in every stream
// -- views of one arena per stream, in order -- become one segment: the
// update is elementwise, so the merged segment computes exactly what its
// parts would, in one launch instead of one per part (a list of views of a
// flattened bucket then launches like the bucket itself).
std::vector<SegDesc> coalesce(const std::vector<SegDesc> &active, int gdt) {
    std::vector<SegDesc> out;
    out.reserve(active.size());
    const int64_t gb = static_cast<int64_t>(grad_bytes(gdt));
    auto follows = [](const void *next, const void *cur, int64_t bytes) {
        return reinterpret_cast<uintptr_t>(next) == reinterpret_cast<uintptr_t>(cur) + static_cast<uintptr_t>(bytes);
    };
    for (const SegDesc &d : active) {
        if (!out.empty()) {
            SegDesc &c = out.back();
            const int64_t fb = c.n * 4;
            bool adj = follows(d.p_out, c.p_out, fb) && follows(d.g, c.g, c.n * gb) && follows(d.m_out, c.m_out, fb) &&
                       follows(d.v_out, c.v_out, fb) && (d.vmax_out == nullptr) == (c.vmax_out == nullptr) &&
                       (d.vmax_out == nullptr || follows(d.vmax_out, c.vmax_out, fb)) && d.model_kind == c.model_kind &&
                       (d.model_kind == 0 || follows(d.model, c.model, c.n * 2));
            if (adj) {
                c.n += d.n;
                continue;
            }
        }
        out.push_back(d);
    }
    return out;
}

// Launch policy: a tensor of at least MULTI_SOLO_MIN elements gets a launch
// of its own; all smaller tensors share one launch.
void split_launches(const std::vector<SegDesc> &active, std::vector<SegDesc> &solo, std::vector<SegDesc> &shared) {
    for (const SegDesc &d : active) (d.n >= MULTI_SOLO_MIN ? solo : shared).push_back(d);
}

// The device's auxiliary update stream and its two events (aux_mu held).
int ensure_aux(DeviceCache &dc, int dev) {
    if (dc.aux) return RADAMW_OK;
    DeviceScope scope(dev);
    hipStream_t s = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_status(e);
    hipEvent_t f = nullptr, j = nullptr;
    e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (e != hipSuccess) {
        if (f) (void)hipEventDestroy(f);
        (void)hipStreamDestroy(s);
        return hip_status(e);
    }
    dc.aux = s;
    dc.fork = f;
    dc.join = j;
    return RADAMW_OK;
}

// Submit the update launches of one step: every solo tensor, then the
// shared ones in one launch, whose table is either staged now or already
// resident in device memory (resident != null: its image and device base).
// With two or more launches, every other one goes to the device's auxiliary
// stream: back-to-back launches on one stream each pay a ramp and a drain
// (~3-4 us on MI355X), which two streams overlap.  The LDS reservation caps
// residency per CU across both, so HBM sees the same bytes in flight.  The
// auxiliary stream first waits for everything queued on `stream` so far
// (the fused step's decision included), and `stream` waits for all of it
// before anything queued after this call.  Measurement events, if
// requested: the start on the first launch, the stop on `stream` after the
// join.
int submit_updates(const std::vector<SegDesc> &solo, std::vector<SegDesc> &shared, const UpdateTable *resident,
                   const char *resident_base, int gdt, bool ams, bool first, const Coefs &c, const Decision *dec,
                   int dev, hipStream_t stream, UpdateTiming timing) {
    const size_t launches = solo.size() + (shared.empty() ? 0 : 1);
    DeviceCache &dc = g_devices[dev];
    std::unique_lock<std::mutex> lock(dc.aux_mu, std::defer_lock);
    const bool two = launches >= 2;
    int rc = RADAMW_OK;
    if (two) {
        lock.lock();
        if ((rc = ensure_aux(dc, dev))) return rc;
        hipError_t e = hipEventRecord(dc.fork, stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(dc.aux, dc.fork, 0);
        if (e != hipSuccess) return hip_status(e);
    }
    size_t k = 0;
    auto on = [&]() { return two && (k & 1) ? dc.aux : stream; };
    auto ev_start = [&]() { return k == 0 ? timing.start : nullptr; };
    auto ev_stop = [&]() { return !two && k + 1 == launches ? timing.stop : nullptr; };
    for (const SegDesc &d : solo) {
        if ((rc = launch_single(d, gdt, ams, first, c, dec, dev, on(), ev_start(), ev_stop()))) break;
        ++k;
    }
    if (rc == RADAMW_OK) {
        if (shared.size() == 1) {
            rc = launch_single(shared[0], gdt, ams, first, c, dec, dev, on(), ev_start(), ev_stop());
        } else if (shared.size() > 1 && resident) {
            rc = hip_status(
                launch_table_at(*resident, resident_base, gdt, ams, first, c, dec, on(), ev_start(), ev_stop()));
            if (rc == RADAMW_OK) g_launches.fetch_add(1, std::memory_order_relaxed);
        } else if (shared.size() > 1) {
            rc = launch_table(shared, gdt, ams, first, c, dec, dev, on(), ev_start(), ev_stop());
        }
    }
    if (two) {
        // join even after a failed launch, so that `stream` still orders
        // after whatever reached the auxiliary stream
        hipError_t e = hipEventRecord(dc.join, dc.aux);
        if (e == hipSuccess) e = hipStreamWaitEvent(stream, dc.join, 0);
        if (e == hipSuccess && rc == RADAMW_OK && timing.stop) e = hipEventRecord(timing.stop, stream);
        if (e != hipSuccess && rc == RADAMW_OK) rc = hip_status(e);
    }
    return rc;
}

// Validated multi-tensor update (shared by radamw_step_multi, the write-back
// variant and the fused step).
int multi_update(const radamw_segment *segs, int32_t nseg, int gdt, uint64_t *step,
                 const radamw_options &o, double gradient_scale, int dev, hipStream_t stream,
                 int32_t *updated, void *const *models = nullptr, int model_dtype = 0) {
    std::vector<SegDesc> active = coalesce(inplace_descs(segs, nseg, models, model_dtype), gdt);
    if (active.empty()) {
        *updated = 0;
        return RADAMW_OK;
    }
    const Coefs c = make_coefs(o, *step + 1, gradient_scale);
    std::vector<SegDesc> solo, shared;
    split_launches(active, solo, shared);
    const UpdateTiming timing = g_timing;
    g_timing = UpdateTiming{};
    const int rc =
        submit_updates(solo, shared, nullptr, nullptr, gdt, o.amsgrad != 0, *step == 0, c, nullptr, dev, stream, timing);
    if (rc != RADAMW_OK) return rc;
    *step += 1;
    *updated = 1;
    return RADAMW_OK;
}

// Validate a segment list for an in-place multi-tensor update (and its
// optional 16-bit model copies, which are written ranges too).
int check_segments(const radamw_segment *segs, int32_t nseg, int gdt, bool amsgrad, bool first,
                   int dev, int64_t *active_out, void *const *models = nullptr) {
    if (nseg < 0 || (nseg > 0 && !segs)) return RADAMW_ERR_INVALID;
    PtrChecker pc(dev);
    std::vector<Range> ranges;
    ranges.reserve(static_cast<size_t>(nseg) * 5);
    int64_t active = 0;
    for (int32_t i = 0; i < nseg; ++i) {
        const radamw_segment &s = segs[i];
        if (s.n < 0) return RADAMW_ERR_INVALID;
        if (s.n > MAX_ELEMENTS) return RADAMW_ERR_RANGE;
        if (s.n == 0) continue;  // empty tensors may carry null pointers
        if ((s.max_exp_avg_sq != nullptr) != amsgrad) return RADAMW_ERR_STATE;
        ++active;
        SegDesc d{};
        d.p_in = d.p_out = s.param;
        d.g = s.grad;
        d.m_in = d.m_out = s.exp_avg;
        d.v_in = d.v_out = s.exp_avg_sq;
        d.vmax_in = d.vmax_out = s.max_exp_avg_sq;
        d.n = s.n;
        int rc = check_update_tensor(d, gdt, amsgrad, first, true, pc, ranges);
        if (rc) return rc;
        if (models && models[i]) {
            if ((rc = pc.check(models[i], 2, s.n * 2))) return rc;
            add_range(ranges, models[i], s.n * 2, true);
        }
    }
    if (active_out) *active_out = active;
    return check_alias(ranges);
}

int64_t stats_rows(int64_t n, int gdt) {
    if (n == 0) return 0;
    const int64_t epc = gdt == RADAMW_F32 ? 4 : 8;
    const int64_t per_row = int64_t(STATS_BLOCK) * STATS_UNROLL * epc;
    return std::min<int64_t>((n + per_row - 1) / per_row, STATS_ROWS_CAP);
}

int32_t stats_head(const void *g, int gdt, int64_t n) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(g);
    int64_t head = static_cast<int64_t>((16 - (a & 15)) & 15) / static_cast<int64_t>(grad_bytes(gdt));
    return static_cast<int32_t>(std::min(head, n));
}

int plan(int64_t rows, int64_t *scratch_elements, int32_t *extra) {
    if (rows < 1 || rows > STATS_MAX_ROWS) return RADAMW_ERR_RANGE;
    int64_t remaining = rows, records = 0;
    int32_t levels = 0;
    while (remaining > MERGE_FAN_IN) {
        remaining = (remaining + MERGE_FAN_IN - 1) / MERGE_FAN_IN;
        records += remaining;
        ++levels;
    }
    *scratch_elements = 3 * records;
    *extra = levels;
    return RADAMW_OK;
}

// The fan-in-1024 levels (hierarchical only) for already validated
// arguments: *cur / *count receive the records the final merge reduces.
int merge_levels(const StatsRec *rows, int64_t nrows, StatsRec *scratch, bool hierarchical, hipStream_t stream,
                 const StatsRec **cur_out, int64_t *count_out) {
    const StatsRec *cur = rows;
    int64_t count = nrows;
    if (hierarchical) {
        StatsRec *level = scratch;
        while (count > MERGE_FAN_IN) {
            const int64_t blocks = (count + MERGE_FAN_IN - 1) / MERGE_FAN_IN;
            int rc = hip_status(launch_merge(cur, count, MERGE_FAN_IN, blocks, level, stream));
            if (rc) return rc;
            g_launches.fetch_add(1, std::memory_order_relaxed);
            cur = level;
            count = blocks;
            level += blocks;
        }
    }
    *cur_out = cur;
    *count_out = count;
    return RADAMW_OK;
}

// Launch the merges for already validated arguments.
int merge_launch(const StatsRec *rows, int64_t nrows, StatsRec *scratch, StatsRec *report,
                 bool hierarchical, hipStream_t stream) {
    const StatsRec *cur;
    int64_t count;
    int rc = merge_levels(rows, nrows, scratch, hierarchical, stream, &cur, &count);
    if (rc) return rc;
    rc = hip_status(launch_merge(cur, count, count, 1, report, stream));
    if (rc) return rc;
    g_launches.fetch_add(1, std::memory_order_relaxed);
    return RADAMW_OK;
}

int read_report(const StatsRec *report, radamw_stats *host, int dev, hipStream_t stream) {
    DeviceCache &dc = g_devices[dev];
    std::lock_guard<std::mutex> lock(dc.mu);
    if (!dc.pinned_report) {
        void *p = nullptr;
        hipError_t e = hipHostMalloc(&p, 64, hipHostMallocDefault);
        if (e != hipSuccess) return hip_status(e);
        dc.pinned_report = static_cast<radamw_stats *>(p);
    }
    hipError_t e = hipMemcpyAsync(dc.pinned_report, report, sizeof(radamw_stats), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return hip_status(e);
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e);
    std::memcpy(host, dc.pinned_report, sizeof(radamw_stats));
    return RADAMW_OK;
}

void decode(const radamw_stats &r, double *sumsq, uint32_t *count) {
    const uint64_t bits = uint64_t(r.w[0]) | (uint64_t(r.w[1]) << 32);
    std::memcpy(sumsq, &bits, sizeof(double));
    *count = r.w[2];
}

// The statistics rows of a list of non-empty gradients, packed back to back
// (the same records per-tensor launches would write).
std::vector<StatsSeg> stats_segments(const radamw_segment *segs, int32_t nseg, int gdt, int64_t *nrows_out) {
    std::vector<StatsSeg> st;
    st.reserve(static_cast<size_t>(nseg));
    int64_t nrows = 0;
    for (int32_t i = 0; i < nseg; ++i) {
        const radamw_segment &s = segs[i];
        if (s.n == 0) continue;
        const int64_t r = stats_rows(s.n, gdt);
        st.push_back(StatsSeg{s.grad, s.n, nrows, stats_head(s.grad, gdt, s.n), static_cast<int32_t>(r)});
        nrows += r;
    }
    *nrows_out = nrows;
    return st;
}

// Device image of a multi-tensor statistics launch: the StatsSeg array,
// then coarse[j] = the gradient holding row j << STATS_COARSE_LOG2 (the last
// entry closes the range with the last gradient).
std::vector<char> build_stats_table(const std::vector<StatsSeg> &st, int64_t nrows, size_t *coarse_off) {
    const int32_t ns = static_cast<int32_t>(st.size());
    const int64_t ncoarse = ((nrows - 1) >> STATS_COARSE_LOG2) + 1;
    std::vector<int32_t> coarse(ncoarse + 1);
    int32_t k = 0;
    for (int64_t j = 0; j < ncoarse; ++j) {
        const int64_t r = j << STATS_COARSE_LOG2;
        while (k + 1 < ns && st[k + 1].row_begin <= r) ++k;
        coarse[j] = k;
    }
    coarse[ncoarse] = ns - 1;
    const size_t seg_bytes = sizeof(StatsSeg) * st.size();
    std::vector<char> bytes(seg_bytes + sizeof(int32_t) * coarse.size());
    std::memcpy(bytes.data(), st.data(), seg_bytes);
    std::memcpy(bytes.data() + seg_bytes, coarse.data(), sizeof(int32_t) * coarse.size());
    *coarse_off = seg_bytes;
    return bytes;
}

// The per-device page of host memory mapped for the device, which receives
// the final merge's report, decision and completion word (report_mu held).
int ensure_mapped(DeviceCache &dc, int dev) {
    if (dc.mapped_report_host) return RADAMW_OK;
    DeviceScope scope(dev);
    void *hp = nullptr, *dp = nullptr;
    hipError_t e = hipHostMalloc(&hp, 64, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) return hip_status(e);
    e = hipHostGetDevicePointer(&dp, hp, 0);
    if (e != hipSuccess) {
        (void)hipHostFree(hp);
        return hip_status(e);
    }
    std::memset(hp, 0, 64);
    dc.mapped_report_host = static_cast<radamw_stats *>(hp);
    dc.mapped_report_dev = static_cast<radamw_stats *>(dp);
    dc.mapped_decision_host = reinterpret_cast<Decision *>(static_cast<char *>(hp) + 16);
    dc.mapped_decision_dev = reinterpret_cast<Decision *>(static_cast<char *>(dp) + 16);
    dc.mapped_done_host = reinterpret_cast<volatile uint32_t *>(static_cast<char *>(hp) + 32);
    dc.mapped_done_dev = reinterpret_cast<uint32_t *>(static_cast<char *>(dp) + 32);
    return RADAMW_OK;
}

// Wait until the final merge of this call has written `seq` to the mapped
// completion word.  The host spins for WAIT_SPIN, then yields its thread
// between reads (a step called with a long backward pass still queued
// would otherwise keep a core busy all along; the GPU has the update
// kernels queued meanwhile, so a late return costs it nothing).  A wait
// longer than WAIT_CHECK_PERIOD also asks the stream, once per period,
// whether it can still get there: an error on the stream, or a stream that
// has drained without the word, ends the wait with an error.  (Asking on
// every wait would cost the GPU time: the runtime answers a query on a busy
// stream by queueing a completion marker behind its last kernel.)
constexpr auto WAIT_SPIN = std::chrono::milliseconds(1);
constexpr auto WAIT_CHECK_PERIOD = std::chrono::milliseconds(10);

int wait_done(const DeviceCache &dc, uint32_t seq, hipStream_t stream) {
    const auto start = std::chrono::steady_clock::now();
    auto next_check = start + WAIT_CHECK_PERIOD;
    bool yield = false;
    for (uint32_t i = 1;; ++i) {
        if (*dc.mapped_done_host == seq) break;
        if (yield)
            std::this_thread::yield();
        else
            __builtin_ia32_pause();
        if ((i & 255) == 0) {
            const auto now = std::chrono::steady_clock::now();
            yield = yield || now - start >= WAIT_SPIN;
            if (now >= next_check) {
                const hipError_t e = hipStreamQuery(stream);
                if (e != hipSuccess && e != hipErrorNotReady) return hip_status(e);
                if (e == hipSuccess && *dc.mapped_done_host != seq) return hip_status(hipErrorUnknown);
                next_check = std::chrono::steady_clock::now() + WAIT_CHECK_PERIOD;
            }
        }
    }
    std::atomic_thread_fence(std::memory_order_acquire);
    return RADAMW_OK;
}

// The tail of every fused step, under the device's report lock:
//   prepare(&cur, &count)  launches whatever merges leave `count` records at
//                          `cur` for the final merge;
//   the final merge reduces them, takes the skip / clip decision on the
//   device and writes report and decision into the mapped page, and the
//   decision also to dec_dev, where the update kernels read it; then it
//   writes this call's sequence number to the page's completion word;
//   submit()               queues the update launches right behind it;
// only then does the host wait, for the merge alone, by watching that word,
// and read the page.  Nothing is queued between the merge and the updates,
// so the GPU goes from one to the other without a gap.
template <typename Prepare, typename Submit>
int fused_tail(int dev, hipStream_t stream, Decision *dec_dev, const DecideArgs &args, radamw_stats *host,
               Decision *host_dec, Prepare prepare, Submit submit) {
    DeviceCache &dc = g_devices[dev];
    std::lock_guard<std::mutex> lock(dc.report_mu);
    int rc = ensure_mapped(dc, dev);
    if (rc) return rc;
    const StatsRec *cur = nullptr;
    int64_t count = 0;
    if ((rc = prepare(&cur, &count))) return rc;
    if (++dc.done_seq == 0) dc.done_seq = 1;  // the page starts at 0
    DecideArgs a = args;
    a.done = dc.mapped_done_dev;
    a.seq = dc.done_seq;
    rc = hip_status(launch_merge_decide(cur, count, reinterpret_cast<StatsRec *>(dc.mapped_report_dev), dec_dev,
                                        dc.mapped_decision_dev, a, stream));
    if (rc) return rc;
    g_launches.fetch_add(1, std::memory_order_relaxed);
    const int submitted = submit();
    if ((rc = wait_done(dc, a.seq, stream))) return rc;
    std::memcpy(host, dc.mapped_report_host, sizeof *host);
    std::memcpy(host_dec, dc.mapped_decision_host, sizeof *host_dec);
    return submitted;
}

// The decision of TR-zh from a report on the host (radamw_decide).
int decide_host(const radamw_stats *host_report, double gradient_scale, double max_grad_norm,
                radamw_control *ctrl, radamw_fused_result *result) {
    if (!host_report || !ctrl || !is_finite(max_grad_norm)) return RADAMW_ERR_INVALID;
    int rc;
    if ((rc = check_scale(gradient_scale))) return rc;
    double sumsq;
    uint32_t count;
    decode(*host_report, &sumsq, &count);
    const double norm = std::sqrt(sumsq) / gradient_scale;
    double clip = 1.0;
    if (max_grad_norm > 0.0) clip = std::min(1.0, max_grad_norm / (norm + 1e-6));
    // a skipped step applies no clip: the scale passes through unchanged
    ctrl->skip_update = count > 0 ? 1 : 0;
    ctrl->gradient_scale = (count > 0 || clip == 1.0) ? gradient_scale : gradient_scale / clip;
    if (result) {
        result->found_inf = count > 0 ? 1 : 0;
        result->nonfinite = count;
        result->reserved = 0;
        result->sumsq = sumsq;
        result->total_norm = norm;
        result->clip_coef = clip;
    }
    return RADAMW_OK;
}

// The host's decision from the report it read, which must be the device's:
// the same skip, and the same FP32 unscale factor for an update.  Fills the
// result from the report, with `updated` from the device's decision (the one
// the queued kernels applied), and *updated likewise; RADAMW_ERR_DECISION
// when the two decisions differ.
int settle(const radamw_stats &host, const Decision &dev_dec, double gradient_scale, double max_grad_norm,
           radamw_fused_result *result, bool *updated) {
    radamw_control ctrl;
    int rc = decide_host(&host, gradient_scale, max_grad_norm, &ctrl, result);
    if (rc) return rc;
    const bool skip = ctrl.skip_update != 0;
    const bool dev_skip = dev_dec.skip != 0;
    const float inv = static_cast<float>(1.0 / ctrl.gradient_scale);
    uint32_t a, b;
    std::memcpy(&a, &inv, 4);
    std::memcpy(&b, &dev_dec.inv_scale, 4);
    result->updated = dev_skip ? 0 : 1;
    *updated = !dev_skip;
    if (skip != dev_skip || (!skip && a != b)) return RADAMW_ERR_DECISION;
    return RADAMW_OK;
}

}  // namespace

// ========================================================= tensor lists ==

// A validated tensor list kept across steps: the launch split, the update
// descriptors and the statistics rows are computed once, and the device
// tables (plus the statistics rows and merge scratch) live in one device
// allocation the list owns.  Steps on one list serialise on its mutex.
struct radamw_list_s {
    std::mutex mu;
    int dev = 0;
    int gdt = 0;
    bool amsgrad = false;
    int64_t active = 0;
    std::vector<SegDesc> solo, shared;
    UpdateTable table;        // image of the shared launch's table (shared.size() > 1)
    std::vector<StatsSeg> st; // statistics rows of the non-empty gradients
    int64_t nrows = 0;
    size_t stats_coarse_off = 0;
    char *mem = nullptr;      // device: [update table][stats table][rows][merge scratch][decision]
    char *staging = nullptr;  // pinned host copy of the tables, the source of their upload
    size_t table_off = 0, stats_off = 0, rows_off = 0, dec_off = 0;
    hipEvent_t done = nullptr;  // recorded after the last launch that reads `mem`
    bool pending = false;
};

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Checks shared by the list's step entry points.
int list_step_checks(radamw_list_s *l, const radamw_options *opts, const uint64_t *step, hipStream_t stream) {
    int rc;
    if ((rc = check_options(opts))) return rc;
    if (!l || !step) return RADAMW_ERR_INVALID;
    if ((opts->amsgrad != 0) != l->amsgrad) return RADAMW_ERR_STATE;
    if (*step == UINT64_MAX) return RADAMW_ERR_STATE;
    int dev;
    if ((rc = stream_device(stream, &dev))) return rc;
    if (dev != l->dev) return RADAMW_ERR_INVALID;
    return RADAMW_OK;
}

// The update launches of one list step (reading `dec` when a fused step
// decides on the device); the caller records the list's event after them.
int list_launch(radamw_list_s *l, uint64_t step, const radamw_options &o, double gradient_scale,
                const Decision *dec, hipStream_t stream, UpdateTiming timing) {
    const Coefs c = make_coefs(o, step + 1, gradient_scale);
    return submit_updates(l->solo, l->shared, l->shared.size() > 1 ? &l->table : nullptr, l->mem + l->table_off,
                          l->gdt, l->amsgrad, step == 0, c, dec, l->dev, stream, timing);
}

// Record the event that guards the list's memory after its last launch.
int list_mark(radamw_list_s *l, hipStream_t stream) {
    hipError_t e = hipEventRecord(l->done, stream);
    if (e != hipSuccess) return hip_status(e);
    l->pending = true;
    return RADAMW_OK;
}

Decision *list_decision(radamw_list_s *l) { return reinterpret_cast<Decision *>(l->mem + l->dec_off); }

StatsRec *list_rows(radamw_list_s *l) { return reinterpret_cast<StatsRec *>(l->mem + l->rows_off); }

// Order a step after the list's previous work (the table upload, the last
// update), which may have gone to another stream.
int list_wait(radamw_list_s *l, hipStream_t stream) {
    if (!l->pending) return RADAMW_OK;
    return hip_status(hipStreamWaitEvent(stream, l->done, 0));
}

// The analysis launch of a list (its rows go to the list's own memory).
int list_analyze(radamw_list_s *l, hipStream_t stream) {
    int rc;
    if (l->st.size() == 1) {
        const StatsSeg &g = l->st[0];
        rc = hip_status(launch_analyze(g.g, l->gdt, g.n, g.head, g.rows, list_rows(l), stream));
    } else {
        const char *base = l->mem + l->stats_off;
        rc = hip_status(launch_analyze_table(reinterpret_cast<const StatsSeg *>(base),
                                             reinterpret_cast<const int32_t *>(base + l->stats_coarse_off),
                                             l->nrows, l->gdt, list_rows(l), stream));
    }
    if (rc == RADAMW_OK) g_launches.fetch_add(1, std::memory_order_relaxed);
    return rc;
}

}  // namespace

// ===================================================================== ABI ==

extern "C" {

radamw_options radamw_options_default(void) {
    radamw_options o;
    o.lr = 1e-3;
    o.beta1 = 0.9;
    o.beta2 = 0.999;
    o.eps = 1e-5;
    o.weight_decay = 1e-4;
    o.amsgrad = 0;
    o.maximize = 0;
    return o;
}

int radamw_host_coefficients(const radamw_options *opts, uint64_t t, double gradient_scale,
                             float *out9) {
    int rc;
    if ((rc = check_options(opts))) return rc;
    if ((rc = check_scale(gradient_scale))) return rc;
    if (!out9 || t == 0) return RADAMW_ERR_INVALID;
    const Coefs c = make_coefs(*opts, t, gradient_scale);
    const float v[9] = {c.beta1, c.one_minus_beta1, c.beta2, c.one_minus_beta2, c.inv_scale,
                        c.decay, c.step_size, c.inv_bc2, c.eps};
    std::memcpy(out9, v, sizeof v);
    return RADAMW_OK;
}

int radamw_step(const float *p, const void *g, radamw_dtype gdt, int64_t n, const radamw_state *in,
                float *p_out, radamw_state *out, const radamw_options *opts,
                const radamw_control *ctrl, radamw_stream_t stream_, int32_t *updated) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc;
    if ((rc = check_options(opts))) return rc;
    if ((rc = check_control(ctrl))) return rc;
    if (!valid_dtype(gdt) || n < 0 || !in || !out || !updated) return RADAMW_ERR_INVALID;
    if (n > MAX_ELEMENTS) return RADAMW_ERR_RANGE;
    const bool ams = opts->amsgrad != 0;
    const bool first = in->step == 0;
    if (in->step == UINT64_MAX) return RADAMW_ERR_STATE;
    if (n > 0) {
        if ((out->max_exp_avg_sq != nullptr) != ams) return RADAMW_ERR_STATE;
        if (!first && (in->max_exp_avg_sq != nullptr) != ams) return RADAMW_ERR_STATE;
        int dev;
        if ((rc = stream_device(stream, &dev))) return rc;
        SegDesc d{};
        d.p_in = p;
        d.g = g;
        d.m_in = in->exp_avg;
        d.v_in = in->exp_avg_sq;
        d.vmax_in = in->max_exp_avg_sq;
        d.p_out = p_out;
        d.m_out = out->exp_avg;
        d.v_out = out->exp_avg_sq;
        d.vmax_out = out->max_exp_avg_sq;
        d.n = n;
        std::vector<Range> ranges;
        PtrChecker pc(dev);
        if ((rc = check_update_tensor(d, gdt, ams, first, false, pc, ranges))) return rc;
        if ((rc = check_alias(ranges))) return rc;
        if (ctrl->skip_update) {
            *updated = 0;
            return RADAMW_OK;
        }
        const Coefs c = make_coefs(*opts, in->step + 1, ctrl->gradient_scale);
        const UpdateTiming timing = g_timing;
        g_timing = UpdateTiming{};
        if ((rc = launch_single(d, gdt, ams, first, c, nullptr, dev, stream, timing.start, timing.stop))) return rc;
        out->step = in->step + 1;
        *updated = 1;
        return RADAMW_OK;
    }
    *updated = 0;
    return RADAMW_OK;
}

int radamw_step_inplace(float *p, const void *g, radamw_dtype gdt, int64_t n, radamw_state *st,
                        const radamw_options *opts, const radamw_control *ctrl,
                        radamw_stream_t stream_, int32_t *updated) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc;
    if ((rc = check_options(opts))) return rc;
    if ((rc = check_control(ctrl))) return rc;
    if (!valid_dtype(gdt) || n < 0 || !st || !updated) return RADAMW_ERR_INVALID;
    if (n > MAX_ELEMENTS) return RADAMW_ERR_RANGE;
    if (st->step == UINT64_MAX) return RADAMW_ERR_STATE;
    const bool ams = opts->amsgrad != 0;
    if (n == 0) {
        *updated = 0;
        return RADAMW_OK;
    }
    if ((st->max_exp_avg_sq != nullptr) != ams) return RADAMW_ERR_STATE;
    int dev;
    if ((rc = stream_device(stream, &dev))) return rc;
    radamw_segment s{p, g, st->exp_avg, st->exp_avg_sq, st->max_exp_avg_sq, n};
    if ((rc = check_segments(&s, 1, gdt, ams, st->step == 0, dev, nullptr))) return rc;
    if (ctrl->skip_update) {
        *updated = 0;
        return RADAMW_OK;
    }
    return multi_update(&s, 1, gdt, &st->step, *opts, ctrl->gradient_scale, dev, stream, updated);
}

int radamw_step_staged_inplace(float *p, const void *g, radamw_dtype gdt, int64_t n, radamw_state *st,
                               float *delta, const radamw_options *opts, const radamw_control *ctrl,
                               radamw_stream_t stream_, int32_t *updated) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc;
    if ((rc = check_options(opts))) return rc;
    if ((rc = check_control(ctrl))) return rc;
    if (!valid_dtype(gdt) || n < 0 || !st || !updated) return RADAMW_ERR_INVALID;
    if (n > MAX_ELEMENTS) return RADAMW_ERR_RANGE;
    if (st->step == UINT64_MAX) return RADAMW_ERR_STATE;
    const bool ams = opts->amsgrad != 0;
    if (n == 0) {
        *updated = 0;
        return RADAMW_OK;
    }
    if ((st->max_exp_avg_sq != nullptr) != ams) return RADAMW_ERR_STATE;
    int dev;
    if ((rc = stream_device(stream, &dev))) return rc;
    const int64_t fb = n * 4, gb = n * static_cast<int64_t>(grad_bytes(gdt));
    PtrChecker pc(dev);
    // every stream is read in 16-byte chunks (8-byte for 16-bit gradients)
    if ((rc = pc.check(p, 16, fb)) || (rc = pc.check(g, 4 * grad_bytes(gdt), gb)) ||
        (rc = pc.check(st->exp_avg, 16, fb)) || (rc = pc.check(st->exp_avg_sq, 16, fb)) ||
        (rc = pc.check(delta, 16, fb)) || (ams && (rc = pc.check(st->max_exp_avg_sq, 16, fb))))
        return rc;
    std::vector<Range> ranges;
    add_range(ranges, g, gb, false);
    add_range(ranges, p, fb, true);
    add_range(ranges, st->exp_avg, fb, true);
    add_range(ranges, st->exp_avg_sq, fb, true);
    add_range(ranges, delta, fb, true);
    if (ams) add_range(ranges, st->max_exp_avg_sq, fb, true);
    if ((rc = check_alias(ranges))) return rc;
    if ((n >> 2) + (n & 3) > UPDATE_MAX_GRID * 64) return RADAMW_ERR_RANGE;
    if (ctrl->skip_update) {
        *updated = 0;
        return RADAMW_OK;
    }
    const Coefs c = make_coefs(*opts, st->step + 1, ctrl->gradient_scale);
    int launched = 0;
    hipError_t e = launch_staged(p, g, gdt, st->exp_avg, st->exp_avg_sq, ams ? st->max_exp_avg_sq : nullptr,
                                 delta, n, st->step == 0, c, stream, &launched);
    g_launches.fetch_add(static_cast<uint64_t>(launched), std::memory_order_relaxed);
    if (e != hipSuccess) return hip_status(e);
    st->step += 1;
    *updated = 1;
    return RADAMW_OK;
}

int radamw_bucket_layout(int64_t n, const int32_t *element_bytes, int32_t nstreams, int64_t *offsets,
                         int64_t *arena_bytes) {
    if (!element_bytes || !offsets || !arena_bytes || nstreams < 1 || nstreams > 16 || n < 0)
        return RADAMW_ERR_INVALID;
    if (n > MAX_ELEMENTS) return RADAMW_ERR_RANGE;
    int64_t widest = 0;
    for (int32_t k = 0; k < nstreams; ++k) {
        const int32_t e = element_bytes[k];
        if (e != 1 && e != 2 && e != 4 && e != 8) return RADAMW_ERR_INVALID;
        widest = std::max<int64_t>(widest, e);
    }
    const int64_t pitch =
        (n * widest + BUCKET_PITCH_ALIGN - 1) / BUCKET_PITCH_ALIGN * BUCKET_PITCH_ALIGN + BUCKET_STREAM_SHIFT;
    for (int32_t k = 0; k < nstreams; ++k) offsets[k] = k * pitch;
    *arena_bytes = nstreams * pitch;
    return RADAMW_OK;
}

int radamw_stream_probe(const float *const *in, int32_t nreads, float *const *out, int32_t nwrites,
                        int64_t n, int32_t cap_per_cu, radamw_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (nreads < 0 || nreads > 5 || nwrites < 0 || nwrites > 4 || nreads + nwrites < 1) return RADAMW_ERR_INVALID;
    if (cap_per_cu < 0 || cap_per_cu > MAX_WAVES_PER_CU || n < 0) return RADAMW_ERR_INVALID;
    if ((nreads > 0 && !in) || !out) return RADAMW_ERR_INVALID;
    if (n > MAX_ELEMENTS) return RADAMW_ERR_RANGE;
    if (n % 4 != 0) return RADAMW_ERR_ALIGN;
    if (n == 0) return RADAMW_OK;
    if ((n / 4 + 63) / 64 > UPDATE_MAX_GRID) return RADAMW_ERR_RANGE;
    int dev, rc;
    if ((rc = stream_device(stream, &dev))) return rc;
    PtrChecker pc(dev);
    std::vector<Range> ranges;
    ProbeArgs a{};
    // an output that is exactly an input is updated in place (each element
    // is loaded before the same lane stores it); its range counts as written
    auto in_place = [&](const float *q) {
        for (int32_t w = 0; w < nwrites; ++w)
            if (out[w] == q) return true;
        return false;
    };
    for (int32_t r = 0; r < nreads; ++r) {
        if ((rc = pc.check(in[r], 16, n * 4))) return rc;
        if (!in_place(in[r])) add_range(ranges, in[r], n * 4, false);
        a.in[r] = in[r];
    }
    for (int32_t w = 0; w < std::max(nwrites, 1); ++w) {
        if ((rc = pc.check(out[w], 16, n * 4))) return rc;
        add_range(ranges, out[w], n * 4, true);
        a.out[w] = out[w];
    }
    if ((rc = check_alias(ranges))) return rc;
    a.chunks = n / 4;
    a.sink_key = std::numeric_limits<float>::quiet_NaN();
    const UpdateTiming timing = g_timing;
    g_timing = UpdateTiming{};
    rc = hip_status(launch_stream_probe(a, nreads, nwrites, cap_per_cu, stream, timing.start, timing.stop));
    if (rc == RADAMW_OK) g_launches.fetch_add(1, std::memory_order_relaxed);
    return rc;
}

int radamw_step_multi(const radamw_segment *segs, int32_t nseg, radamw_dtype gdt, uint64_t *step,
                      const radamw_options *opts, const radamw_control *ctrl,
                      radamw_stream_t stream_, int32_t *updated) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc;
    if ((rc = check_options(opts))) return rc;
    if ((rc = check_control(ctrl))) return rc;
    if (!valid_dtype(gdt) || !step || !updated) return RADAMW_ERR_INVALID;
    if (*step == UINT64_MAX) return RADAMW_ERR_STATE;
    int dev;
    if ((rc = stream_device(stream, &dev))) return rc;
    int64_t active = 0;
    if ((rc = check_segments(segs, nseg, gdt, opts->amsgrad != 0, *step == 0, dev, &active))) return rc;
    if (ctrl->skip_update || active == 0) {
        *updated = 0;
        return RADAMW_OK;
    }
    return multi_update(segs, nseg, gdt, step, *opts, ctrl->gradient_scale, dev, stream, updated);
}

int radamw_step_multi_writeback(const radamw_segment *segs, void *const *models, int32_t nseg,
                                radamw_dtype gdt, radamw_dtype model_dtype, uint64_t *step,
                                const radamw_options *opts, const radamw_control *ctrl,
                                radamw_stream_t stream_, int32_t *updated) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc;
    if ((rc = check_options(opts))) return rc;
    if ((rc = check_control(ctrl))) return rc;
    if (!valid_dtype(gdt) || !step || !updated) return RADAMW_ERR_INVALID;
    if (model_dtype != RADAMW_F16 && model_dtype != RADAMW_BF16) return RADAMW_ERR_INVALID;
    if (nseg > 0 && !models) return RADAMW_ERR_INVALID;
    if (*step == UINT64_MAX) return RADAMW_ERR_STATE;
    int dev;
    if ((rc = stream_device(stream, &dev))) return rc;
    int64_t active = 0;
    if ((rc = check_segments(segs, nseg, gdt, opts->amsgrad != 0, *step == 0, dev, &active, models))) return rc;
    if (ctrl->skip_update || active == 0) {
        *updated = 0;
        return RADAMW_OK;
    }
    return multi_update(segs, nseg, gdt, step, *opts, ctrl->gradient_scale, dev, stream, updated, models,
                        model_dtype);
}

int radamw_stats_plan(int64_t rows, int64_t *scratch_elements, int32_t *extra_merge_kernels) {
    if (!scratch_elements || !extra_merge_kernels) return RADAMW_ERR_INVALID;
    int64_t se;
    int32_t ex;
    int rc = plan(rows, &se, &ex);
    if (rc) return rc;
    *scratch_elements = se;
    *extra_merge_kernels = ex;
    return RADAMW_OK;
}

int64_t radamw_grad_stats_rows(int64_t n, radamw_dtype gdt) {
    if (n < 0 || !valid_dtype(gdt)) return RADAMW_ERR_INVALID;
    if (n > MAX_ELEMENTS) return RADAMW_ERR_RANGE;
    return stats_rows(n, gdt);
}

int radamw_grad_stats(const void *g, radamw_dtype gdt, int64_t n, radamw_stats *rows_out,
                      int64_t rows_capacity, int64_t *rows_written, radamw_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!valid_dtype(gdt) || n < 0 || !rows_written || rows_capacity < 0) return RADAMW_ERR_INVALID;
    if (n > MAX_ELEMENTS) return RADAMW_ERR_RANGE;
    const int64_t rows = stats_rows(n, gdt);
    if (rows == 0) {
        *rows_written = 0;
        return RADAMW_OK;
    }
    if (rows_capacity < rows) return RADAMW_ERR_RANGE;
    int dev, rc;
    if ((rc = stream_device(stream, &dev))) return rc;
    PtrChecker pc(dev);
    if ((rc = pc.check(g, grad_bytes(gdt), n * static_cast<int64_t>(grad_bytes(gdt))))) return rc;
    if ((rc = pc.check(rows_out, 4, rows * 12))) return rc;
    std::vector<Range> ranges;
    add_range(ranges, g, n * static_cast<int64_t>(grad_bytes(gdt)), false);
    add_range(ranges, rows_out, rows * 12, true);
    if ((rc = check_alias(ranges))) return rc;
    rc = hip_status(launch_analyze(g, gdt, n, stats_head(g, gdt, n), rows,
                                   reinterpret_cast<StatsRec *>(rows_out), stream));
    if (rc) return rc;
    g_launches.fetch_add(1, std::memory_order_relaxed);
    *rows_written = rows;
    return RADAMW_OK;
}

int radamw_merge_stats(const radamw_stats *rows, int64_t nrows, float *scratch,
                       int64_t scratch_elements, radamw_stats *report, int32_t hierarchical,
                       radamw_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (hierarchical != 0 && hierarchical != 1) return RADAMW_ERR_INVALID;
    int64_t need;
    int32_t extra;
    int rc = plan(nrows, &need, &extra);
    if (rc) return rc;
    if (!hierarchical) need = 0;
    if (scratch_elements < need || scratch_elements < 0) return RADAMW_ERR_RANGE;
    int dev;
    if ((rc = stream_device(stream, &dev))) return rc;
    PtrChecker pc(dev);
    if ((rc = pc.check(rows, 4, nrows * 12))) return rc;
    if ((rc = pc.check(report, 4, 12))) return rc;
    if (need > 0 && (rc = pc.check(scratch, 4, need * 4))) return rc;
    std::vector<Range> ranges;
    add_range(ranges, rows, nrows * 12, false);
    add_range(ranges, report, 12, true);
    add_range(ranges, scratch, need * 4, true);
    if ((rc = check_alias(ranges))) return rc;
    return merge_launch(reinterpret_cast<const StatsRec *>(rows), nrows,
                        reinterpret_cast<StatsRec *>(scratch), reinterpret_cast<StatsRec *>(report),
                        hierarchical != 0, stream);
}

int radamw_read_report(const radamw_stats *report, radamw_stats *host_report, radamw_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!host_report) return RADAMW_ERR_INVALID;
    int dev, rc;
    if ((rc = stream_device(stream, &dev))) return rc;
    PtrChecker pc(dev);
    if ((rc = pc.check(report, 4, 12))) return rc;
    return read_report(reinterpret_cast<const StatsRec *>(report), host_report, dev, stream);
}

int radamw_decide(const radamw_stats *host_report, double gradient_scale, double max_grad_norm,
                  radamw_control *ctrl, radamw_fused_result *result) {
    return decide_host(host_report, gradient_scale, max_grad_norm, ctrl, result);
}

int radamw_check_decision(const radamw_stats *host_report, const uint32_t *device_decision,
                          double gradient_scale, double max_grad_norm, radamw_fused_result *result) {
    if (!host_report || !device_decision || !result) return RADAMW_ERR_INVALID;
    Decision d;
    d.skip = device_decision[0];
    std::memcpy(&d.inv_scale, &device_decision[1], 4);
    bool updated = false;
    return settle(*host_report, d, gradient_scale, max_grad_norm, result, &updated);
}

int64_t radamw_fused_workspace_bytes(const radamw_segment *segs, int32_t nseg, radamw_dtype gdt) {
    if (nseg < 0 || (nseg > 0 && !segs) || !valid_dtype(gdt)) return RADAMW_ERR_INVALID;
    int64_t rows = 0;
    for (int32_t i = 0; i < nseg; ++i) {
        if (segs[i].n < 0) return RADAMW_ERR_INVALID;
        if (segs[i].n > MAX_ELEMENTS) return RADAMW_ERR_RANGE;
        rows += stats_rows(segs[i].n, gdt);
    }
    if (rows == 0) return 0;
    int64_t se;
    int32_t ex;
    int rc = plan(rows, &se, &ex);
    if (rc) return rc;
    return rows * 12 + se * 4 + 12;
}

int radamw_fused_step_multi(const radamw_segment *segs, int32_t nseg, radamw_dtype gdt,
                            uint64_t *step, const radamw_options *opts, double gradient_scale,
                            double max_grad_norm, int32_t hierarchical, void *workspace,
                            int64_t workspace_bytes, radamw_stream_t stream_,
                            radamw_fused_result *result) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc;
    if ((rc = check_options(opts))) return rc;
    if ((rc = check_scale(gradient_scale))) return rc;
    if (!valid_dtype(gdt) || !step || !result || !is_finite(max_grad_norm)) return RADAMW_ERR_INVALID;
    if (hierarchical != 0 && hierarchical != 1) return RADAMW_ERR_INVALID;
    if (*step == UINT64_MAX) return RADAMW_ERR_STATE;
    int dev;
    if ((rc = stream_device(stream, &dev))) return rc;
    int64_t active = 0;
    if ((rc = check_segments(segs, nseg, gdt, opts->amsgrad != 0, *step == 0, dev, &active))) return rc;
    const int64_t need = radamw_fused_workspace_bytes(segs, nseg, gdt);
    if (need < 0) return static_cast<int>(need);
    std::memset(result, 0, sizeof *result);
    result->clip_coef = 1.0;
    if (active == 0) return RADAMW_OK;
    if (workspace_bytes < need) return RADAMW_ERR_RANGE;
    {
        PtrChecker pc(dev);
        if ((rc = pc.check(workspace, 8, need))) return rc;
    }
    {
        // the workspace is written; it may overlap no tensor of the step
        std::vector<Range> ranges;
        add_range(ranges, workspace, need, true);
        for (int32_t i = 0; i < nseg; ++i) {
            const radamw_segment &s = segs[i];
            add_range(ranges, s.grad, s.n * static_cast<int64_t>(grad_bytes(gdt)), false);
            add_range(ranges, s.param, s.n * 4, false);
            add_range(ranges, s.exp_avg, s.n * 4, false);
            add_range(ranges, s.exp_avg_sq, s.n * 4, false);
            add_range(ranges, s.max_exp_avg_sq, s.n * 4, false);
        }
        if ((rc = check_alias(ranges))) return rc;
    }

    // statistics of every active gradient, rows packed back to back in one
    // launch (the same records per-tensor launches would write)
    StatsRec *rows = static_cast<StatsRec *>(workspace);
    int64_t nrows = 0;
    const std::vector<StatsSeg> st = stats_segments(segs, nseg, gdt, &nrows);
    if (st.size() == 1) {
        rc = hip_status(launch_analyze(st[0].g, gdt, st[0].n, st[0].head, st[0].rows, rows, stream));
        if (rc) return rc;
        g_launches.fetch_add(1, std::memory_order_relaxed);
    } else {
        size_t coarse_off = 0;
        const std::vector<char> table = build_stats_table(st, nrows, &coarse_off);
        rc = staged_launch(
            dev, stream, table.size(), [&](char *host) { std::memcpy(host, table.data(), table.size()); },
            [&](const char *dev_base) {
                return launch_analyze_table(reinterpret_cast<const StatsSeg *>(dev_base),
                                            reinterpret_cast<const int32_t *>(dev_base + coarse_off), nrows, gdt,
                                            rows, stream);
            });
        if (rc) return rc;
    }
    // the update launches are queued behind the final merge and read its
    // decision from the workspace's last 12 bytes
    // the 8-byte decision, 8-byte aligned inside the workspace's last 12 bytes
    const int64_t dec_off = (need - 12) % 8 == 0 ? need - 12 : need - 8;
    Decision *dec_dev = reinterpret_cast<Decision *>(static_cast<char *>(workspace) + dec_off);
    std::vector<SegDesc> solo, shared;
    split_launches(coalesce(inplace_descs(segs, nseg, nullptr, 0), gdt), solo, shared);
    const Coefs c = make_coefs(*opts, *step + 1, gradient_scale);
    const UpdateTiming timing = g_timing;
    g_timing = UpdateTiming{};
    radamw_stats host;
    Decision dd;
    rc = fused_tail(
        dev, stream, dec_dev, DecideArgs{gradient_scale, max_grad_norm}, &host, &dd,
        [&](const StatsRec **cur, int64_t *count) {
            return merge_levels(rows, nrows, rows + nrows, hierarchical != 0, stream, cur, count);
        },
        [&]() {
            return submit_updates(solo, shared, nullptr, nullptr, gdt, opts->amsgrad != 0, *step == 0, c, dec_dev,
                                  dev, stream, timing);
        });
    if (rc) return rc;
    bool updated = false;
    rc = settle(host, dd, gradient_scale, max_grad_norm, result, &updated);
    if (rc != RADAMW_OK && rc != RADAMW_ERR_DECISION) return rc;
    if (updated) *step += 1;
    return rc;
}

int radamw_fused_step_multi_noalloc(const radamw_segment *segs, int32_t nseg, radamw_dtype gdt, uint64_t *step,
                                    const radamw_options *opts, double gradient_scale, double max_grad_norm,
                                    int32_t hierarchical, radamw_stream_t stream_, radamw_fused_result *result) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc;
    if ((rc = check_options(opts))) return rc;
    if ((rc = check_scale(gradient_scale))) return rc;
    if (!valid_dtype(gdt) || !step || !result || !is_finite(max_grad_norm)) return RADAMW_ERR_INVALID;
    if (hierarchical != 0 && hierarchical != 1) return RADAMW_ERR_INVALID;
    if (nseg < 0 || (nseg > 0 && !segs)) return RADAMW_ERR_INVALID;
    if (nseg > 1) return RADAMW_ERR_RANGE;  // one flattened bucket at most
    if (*step == UINT64_MAX) return RADAMW_ERR_STATE;
    int dev;
    if ((rc = stream_device(stream, &dev))) return rc;
    int64_t active = 0;
    if ((rc = check_segments(segs, nseg, gdt, opts->amsgrad != 0, *step == 0, dev, &active))) return rc;
    const int64_t need = radamw_fused_workspace_bytes(segs, nseg, gdt);
    if (need < 0) return static_cast<int>(need);
    if (need > NOALLOC_WORKSPACE_BYTES) return RADAMW_ERR_RANGE;
    std::memset(result, 0, sizeof *result);
    result->clip_coef = 1.0;
    if (active == 0) return RADAMW_OK;

    DeviceCache &dc = g_devices[dev];
    std::lock_guard<std::mutex> lock(dc.noalloc_mu);  // held until the step has completed
    if (!dc.noalloc_scratch) {
        // set-up, once per device, with that device current: `scratch` names
        // a host-side stand-in; its device copy lives at this address
        DeviceScope scope(dev);
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
        dc.noalloc_scratch = static_cast<char *>(ptr);
    }
    char *ws = dc.noalloc_scratch;
    const radamw_segment &seg = segs[0];
    StatsRec *rows = reinterpret_cast<StatsRec *>(ws);
    const int64_t nrows = stats_rows(seg.n, gdt);
    rc = hip_status(launch_analyze(seg.grad, gdt, seg.n, stats_head(seg.grad, gdt, seg.n), nrows, rows, stream));
    if (rc) return rc;
    g_launches.fetch_add(1, std::memory_order_relaxed);
    const StatsRec *cur = nullptr;
    int64_t count = 0;
    if ((rc = merge_levels(rows, nrows, rows + nrows, hierarchical != 0, stream, &cur, &count))) return rc;
    // the decision slot where a workspace of `need` bytes keeps it
    const int64_t dec_off = (need - 12) % 8 == 0 ? need - 12 : need - 8;
    Decision *dec_dev = reinterpret_cast<Decision *>(ws + dec_off);
    StatsRec *report = reinterpret_cast<StatsRec *>(ws + NOALLOC_REPORT_OFF);
    Decision *dec_copy = reinterpret_cast<Decision *>(ws + NOALLOC_DEC_COPY_OFF);
    rc = hip_status(launch_merge_decide(cur, count, report, dec_dev, dec_copy,
                                        DecideArgs{gradient_scale, max_grad_norm}, stream));
    if (rc) return rc;
    g_launches.fetch_add(1, std::memory_order_relaxed);
    // one segment: one update launch on `stream` (no second stream, no table)
    std::vector<SegDesc> solo, shared;
    split_launches(inplace_descs(segs, nseg, nullptr, 0), solo, shared);
    const Coefs c = make_coefs(*opts, *step + 1, gradient_scale);
    const UpdateTiming timing = g_timing;
    g_timing = UpdateTiming{};
    if ((rc = submit_updates(solo, shared, nullptr, nullptr, gdt, opts->amsgrad != 0, *step == 0, c, dec_dev, dev,
                             stream, timing)))
        return rc;
    // the report and the device's decision, read back behind the update
    uint32_t back[6];
    hipError_t e = hipMemcpyAsync(back, ws + NOALLOC_REPORT_OFF, sizeof back, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e);
    radamw_stats host;
    std::memcpy(host.w, back, 12);
    Decision dd;
    std::memcpy(&dd, back + 4, sizeof dd);
    bool updated = false;
    rc = settle(host, dd, gradient_scale, max_grad_norm, result, &updated);
    if (rc != RADAMW_OK && rc != RADAMW_ERR_DECISION) return rc;
    if (updated) *step += 1;
    return rc;
}

int radamw_list_create(const radamw_segment *segs, int32_t nseg, radamw_dtype gdt, int32_t amsgrad,
                       void *const *models, radamw_dtype model_dtype, radamw_stream_t stream_,
                       radamw_list *list_out) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!list_out || nseg < 0 || (nseg > 0 && !segs) || !valid_dtype(gdt)) return RADAMW_ERR_INVALID;
    if (amsgrad != 0 && amsgrad != 1) return RADAMW_ERR_INVALID;
    if (models && model_dtype != RADAMW_F16 && model_dtype != RADAMW_BF16) return RADAMW_ERR_INVALID;
    for (int32_t i = 0; i < nseg; ++i) {
        if (segs[i].n < 0) return RADAMW_ERR_INVALID;
        if (segs[i].n > MAX_ELEMENTS) return RADAMW_ERR_RANGE;
    }
    int rc, dev;
    if ((rc = stream_device(stream, &dev))) return rc;
    int64_t active = 0;
    if ((rc = check_segments(segs, nseg, gdt, amsgrad != 0, false, dev, &active, models))) return rc;

    std::unique_ptr<radamw_list_s> l(new radamw_list_s);
    l->dev = dev;
    l->gdt = gdt;
    l->amsgrad = amsgrad != 0;
    l->active = active;
    std::vector<SegDesc> descs = coalesce(inplace_descs(segs, nseg, models, model_dtype), gdt);
    split_launches(descs, l->solo, l->shared);
    // heads of an in-place update do not depend on the step, so one table
    // serves the first step and every later one
    if (l->shared.size() > 1 && (rc = build_update_table(l->shared, gdt, l->amsgrad, false, &l->table))) return rc;
    l->st = stats_segments(segs, nseg, gdt, &l->nrows);
    int64_t se = 0;
    int32_t ex = 0;
    if (l->nrows > 0 && (rc = plan(l->nrows, &se, &ex))) return rc;
    std::vector<char> stats_table;
    if (l->st.size() > 1) stats_table = build_stats_table(l->st, l->nrows, &l->stats_coarse_off);

    l->table_off = 0;
    l->stats_off = align_up(l->table.bytes.size(), 256);
    l->rows_off = align_up(l->stats_off + stats_table.size(), 256);
    l->dec_off = align_up(l->rows_off + static_cast<size_t>(l->nrows) * 12 + static_cast<size_t>(se) * 4, 16);
    const size_t total = l->dec_off + 16;
    DeviceScope scope(dev);
    bool copying = false;
    auto fail = [&](hipError_t e) {
        if (copying) (void)hipStreamSynchronize(stream);
        if (l->mem) (void)hipFree(l->mem);
        if (l->staging) (void)hipHostFree(l->staging);
        if (l->done) (void)hipEventDestroy(l->done);
        return hip_status(e);
    };
    hipError_t e = hipEventCreateWithFlags(&l->done, hipEventDisableTiming);
    if (e != hipSuccess) {
        l->done = nullptr;
        return fail(e);
    }
    if (total > 0 && (e = hipMalloc(&l->mem, total)) != hipSuccess) {
        l->mem = nullptr;
        return fail(e);
    }
    // the tables go up from pinned memory the list keeps, so creation does
    // not wait for the stream; the event guards both buffers
    const size_t table_bytes = l->stats_off + stats_table.size();
    if (table_bytes > 0) {
        if ((e = hipHostMalloc(&l->staging, table_bytes, hipHostMallocDefault)) != hipSuccess) {
            l->staging = nullptr;
            return fail(e);
        }
        std::memcpy(l->staging + l->table_off, l->table.bytes.data(), l->table.bytes.size());
        std::memcpy(l->staging + l->stats_off, stats_table.data(), stats_table.size());
        copying = true;
        if ((e = hipMemcpyAsync(l->mem, l->staging, table_bytes, hipMemcpyHostToDevice, stream)) != hipSuccess)
            return fail(e);
        if ((e = hipEventRecord(l->done, stream)) != hipSuccess) return fail(e);
        l->pending = true;
    }
    *list_out = l.release();
    return RADAMW_OK;
}

int radamw_list_step(radamw_list list, uint64_t *step, const radamw_options *opts, const radamw_control *ctrl,
                     radamw_stream_t stream_, int32_t *updated) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc;
    if ((rc = check_control(ctrl))) return rc;
    if (!updated) return RADAMW_ERR_INVALID;
    if ((rc = list_step_checks(list, opts, step, stream))) return rc;
    std::lock_guard<std::mutex> lock(list->mu);
    if (ctrl->skip_update || list->active == 0) {
        *updated = 0;
        return RADAMW_OK;
    }
    if ((rc = list_wait(list, stream))) return rc;
    const UpdateTiming timing = g_timing;
    g_timing = UpdateTiming{};
    if ((rc = list_launch(list, *step, *opts, ctrl->gradient_scale, nullptr, stream, timing))) return rc;
    if ((rc = list_mark(list, stream))) return rc;
    *step += 1;
    *updated = 1;
    return RADAMW_OK;
}

int radamw_list_fused_step(radamw_list list, uint64_t *step, const radamw_options *opts, double gradient_scale,
                           double max_grad_norm, int32_t hierarchical, radamw_stream_t stream_,
                           radamw_fused_result *result) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc;
    if ((rc = check_scale(gradient_scale))) return rc;
    if (!result || !is_finite(max_grad_norm)) return RADAMW_ERR_INVALID;
    if (hierarchical != 0 && hierarchical != 1) return RADAMW_ERR_INVALID;
    if ((rc = list_step_checks(list, opts, step, stream))) return rc;
    std::lock_guard<std::mutex> lock(list->mu);
    std::memset(result, 0, sizeof *result);
    result->clip_coef = 1.0;
    if (list->active == 0) return RADAMW_OK;
    if ((rc = list_wait(list, stream))) return rc;
    if ((rc = list_analyze(list, stream))) return rc;
    StatsRec *rows = list_rows(list);
    Decision *dec_dev = list_decision(list);
    const UpdateTiming timing = g_timing;
    g_timing = UpdateTiming{};
    radamw_stats host;
    Decision dd;
    rc = fused_tail(
        list->dev, stream, dec_dev, DecideArgs{gradient_scale, max_grad_norm}, &host, &dd,
        [&](const StatsRec **cur, int64_t *count) {
            return merge_levels(rows, list->nrows, rows + list->nrows, hierarchical != 0, stream, cur, count);
        },
        [&]() {
            int r = list_launch(list, *step, *opts, gradient_scale, dec_dev, stream, timing);
            const int m = list_mark(list, stream);
            return r ? r : m;
        });
    if (rc) return rc;
    bool updated = false;
    rc = settle(host, dd, gradient_scale, max_grad_norm, result, &updated);
    if (rc != RADAMW_OK && rc != RADAMW_ERR_DECISION) return rc;
    if (updated) *step += 1;
    return rc;
}

int radamw_lists_fused_step(const radamw_list *lists, int32_t nlists, uint64_t *steps,
                            const radamw_options *opts, double gradient_scale, double max_grad_norm,
                            int32_t hierarchical, radamw_stream_t stream_, radamw_fused_result *result) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc;
    if (!lists || !steps || !opts || !result || nlists < 1 || nlists > 65536) return RADAMW_ERR_INVALID;
    if ((rc = check_scale(gradient_scale))) return rc;
    if (!is_finite(max_grad_norm)) return RADAMW_ERR_INVALID;
    if (hierarchical != 0 && hierarchical != 1) return RADAMW_ERR_INVALID;
    std::vector<radamw_list_s *> sorted(lists, lists + nlists);
    for (radamw_list_s *l : sorted)
        if (!l) return RADAMW_ERR_INVALID;
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) return RADAMW_ERR_INVALID;
    for (int32_t k = 0; k < nlists; ++k)
        if ((rc = list_step_checks(lists[k], &opts[k], &steps[k], stream))) return rc;
    // every list locked for the whole step, in address order
    std::vector<std::unique_lock<std::mutex>> locks;
    locks.reserve(sorted.size());
    for (radamw_list_s *l : sorted) locks.emplace_back(l->mu);
    std::memset(result, 0, sizeof *result);
    result->clip_coef = 1.0;
    std::vector<int32_t> act;  // lists with at least one non-empty tensor, in call order
    for (int32_t k = 0; k < nlists; ++k)
        if (lists[k]->active > 0) act.push_back(k);
    if (act.empty()) return RADAMW_OK;
    const int dev = lists[act[0]]->dev;
    for (int32_t k : act)
        if ((rc = list_wait(lists[k], stream))) return rc;
    for (int32_t k : act)
        if ((rc = list_analyze(lists[k], stream))) return rc;
    // every list's update reads the decision from the first active list's
    // slot, so every list's event is recorded after the step's last launch
    Decision *dec_dev = list_decision(lists[act[0]]);
    DeviceCache &dc = g_devices[dev];
    const UpdateTiming timing = g_timing;
    g_timing = UpdateTiming{};
    radamw_stats host;
    Decision dd;
    rc = fused_tail(
        dev, stream, dec_dev, DecideArgs{gradient_scale, max_grad_norm}, &host, &dd,
        [&](const StatsRec **cur, int64_t *count) -> int {
            if (act.size() == 1) {
                radamw_list_s *l = lists[act[0]];
                StatsRec *rows = list_rows(l);
                return merge_levels(rows, l->nrows, rows + l->nrows, hierarchical != 0, stream, cur, count);
            }
            // each list's rows reduce to one record; the records, in call
            // order, take the final merge (report_mu is held)
            const int64_t nact = static_cast<int64_t>(act.size());
            if (dc.group_cap < nact) {
                DeviceScope scope(dev);
                if (dc.group_rec) (void)hipFree(dc.group_rec);
                dc.group_rec = nullptr;
                dc.group_cap = 0;
                const int64_t cap = std::max<int64_t>(nact, 256);
                hipError_t e = hipMalloc(&dc.group_rec, static_cast<size_t>(cap) * sizeof(StatsRec));
                if (e != hipSuccess) {
                    dc.group_rec = nullptr;
                    return hip_status(e);
                }
                dc.group_cap = cap;
            }
            for (int64_t i = 0; i < nact; ++i) {
                radamw_list_s *l = lists[act[i]];
                StatsRec *rows = list_rows(l);
                const int r = merge_launch(rows, l->nrows, rows + l->nrows, dc.group_rec + i, hierarchical != 0,
                                           stream);
                if (r) return r;
            }
            *cur = dc.group_rec;
            *count = nact;
            return RADAMW_OK;
        },
        [&]() -> int {
            int r = RADAMW_OK;
            for (size_t i = 0; i < act.size() && r == RADAMW_OK; ++i) {
                const int32_t k = act[i];
                const UpdateTiming t{i == 0 ? timing.start : nullptr, i + 1 == act.size() ? timing.stop : nullptr};
                r = list_launch(lists[k], steps[k], opts[k], gradient_scale, dec_dev, stream, t);
            }
            for (int32_t k : act) {
                const int m = list_mark(lists[k], stream);
                if (r == RADAMW_OK) r = m;
            }
            return r;
        });
    if (rc) return rc;
    bool updated = false;
    rc = settle(host, dd, gradient_scale, max_grad_norm, result, &updated);
    if (rc != RADAMW_OK && rc != RADAMW_ERR_DECISION) return rc;
    if (updated)
        for (int32_t k : act) steps[k] += 1;
    return rc;
}

int radamw_list_destroy(radamw_list list) {
    if (!list) return RADAMW_OK;
    int rc = RADAMW_OK;
    {
        std::lock_guard<std::mutex> lock(list->mu);
        DeviceScope scope(list->dev);
        if (list->pending) {
            hipError_t e = hipEventSynchronize(list->done);
            if (e != hipSuccess) rc = hip_status(e);
        }
        if (list->mem) (void)hipFree(list->mem);
        if (list->staging) (void)hipHostFree(list->staging);
        if (list->done) (void)hipEventDestroy(list->done);
    }
    delete list;
    return rc;
}

const char *radamw_status_string(int status) {
    switch (status) {
    case RADAMW_OK: return "ok (submitted)";
    case RADAMW_ERR_INVALID: return "invalid argument";
    case RADAMW_ERR_STATE: return "optimizer state mismatch";
    case RADAMW_ERR_ALIAS: return "overlapping buffers";
    case RADAMW_ERR_ALIGN: return "misaligned pointer";
    case RADAMW_ERR_RANGE: return "size or capacity out of range";
    case RADAMW_ERR_HIP: return "HIP runtime error";
    case RADAMW_ERR_DECISION: return "host and device decisions differ (the device's was applied)";
    default: return "unknown status";
    }
}

int radamw_last_hip_error(void) { return g_last_hip; }

int radamw_time_next_update(void *start_event, void *stop_event) {
    g_timing.start = static_cast<hipEvent_t>(start_event);
    g_timing.stop = static_cast<hipEvent_t>(stop_event);
    return RADAMW_OK;
}

uint64_t radamw_launch_count(void) { return g_launches.load(std::memory_order_relaxed); }

}  // extern "C"
