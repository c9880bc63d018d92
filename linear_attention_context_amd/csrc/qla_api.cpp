// qla_api.cpp -- the C ABI of libqla.so: argument checks, then one kernel
// launch on the caller's stream.  The operation, the layouts and the error
// contract are documented in include/qla.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "qla.h"
#include "qla_internal.h"

namespace {

bool valid_layout(int v) { return v == QLA_LAYOUT_KV || v == QLA_LAYOUT_VK; }
bool valid_direction(int v) { return v == QLA_DIR_FWD || v == QLA_DIR_BWD; }

// Shape limits: K (a multiple of 16 in [16, 256]) selects a compiled kernel
// family; V is tiled by 16 columns with a ragged last tile handled in 4-float
// vectors.
int check_shape(int batch, int heads, int n_seg, int K, int V)
{
    if (batch < 0 || heads < 0 || n_seg < 0) return QLA_ERR_SHAPE;
    if (K < 16 || K > 256 || K % 16 != 0) return QLA_ERR_SHAPE;
    if (V < 4 || V > 4096 || V % 4 != 0) return QLA_ERR_SHAPE;
    // One workgroup per (chain, column tile): the grid must fit an int, and
    // its work-items (at most 1024 per workgroup) the runtime's 32-bit count.
    const long long chains = (long long)batch * heads;
    const long long groups = chains * qla::tiles_for(V);
    if (groups > INT32_MAX || groups * qla::max_threads_per_group() > (long long)UINT32_MAX) return QLA_ERR_SHAPE;
    return QLA_OK;
}

struct Extent {
    uintptr_t begin, end;
};

Extent extent(const void* p, size_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Extent a, Extent b) { return a.begin < b.end && b.begin < a.end; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The pointer must be device (or managed) memory, and when the runtime knows
// the allocation, [p, p + bytes) must lie inside it.  Errors raised by the
// queries are cleared so that they do not surface in the caller's next check.
int check_memory(const void* p, size_t bytes)
{
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return QLA_ERR_MEMORY;
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return QLA_ERR_MEMORY;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) == hipSuccess) {
        if ((uintptr_t)p + bytes > (uintptr_t)base + size) return QLA_ERR_MEMORY;
    } else {
        (void)hipGetLastError();
    }
    return QLA_OK;
}

// Checks shared by the entry points once the shape is known to be valid and
// the call non-empty: `segments` states of H / M / out in total, `chains`
// initial states.
int check_buffers(const float* H, const float* M, const float* S0, const float* out, long long chains,
                  long long segments, int K, int V)
{
    if (!H || !M || !out) return QLA_ERR_NULL;
    if (!aligned16(H) || !aligned16(M) || !aligned16(out) || (S0 && !aligned16(S0))) return QLA_ERR_ALIGN;
    // Byte counts below must not wrap: 2^40 states of at most 4 MiB each stay
    // within 64 bits (and far beyond any device's memory).
    if (segments > (1LL << 40)) return QLA_ERR_SHAPE;
    const size_t state = (size_t)K * V * sizeof(float);
    const size_t hbytes = (size_t)segments * state;
    const size_t mbytes = (size_t)segments * K * K * sizeof(float);
    const size_t sbytes = (size_t)chains * state;
    const Extent eo = extent(out, hbytes);
    if (out != H && overlap(eo, extent(H, hbytes))) return QLA_ERR_ALIAS;
    if (overlap(eo, extent(M, mbytes))) return QLA_ERR_ALIAS;
    if (S0 && overlap(eo, extent(S0, sbytes))) return QLA_ERR_ALIAS;
    int rc;
    if ((rc = check_memory(H, hbytes)) != QLA_OK) return rc;
    if ((rc = check_memory(M, mbytes)) != QLA_OK) return rc;
    if ((rc = check_memory(out, hbytes)) != QLA_OK) return rc;
    if (S0 && (rc = check_memory(S0, sbytes)) != QLA_OK) return rc;
    return QLA_OK;
}

// Compute units of the current device, queried once per device (an
// immutable property: a racing first query stores the same value).
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The launchers report failure through the thread's last runtime error
// (hipGetLastError after the launch): clear whatever an earlier, unrelated
// call left there first, so that it is not taken for a failed launch.
void clear_stale_error() { (void)hipGetLastError(); }

#if defined(QLA_DEBUG_DELAY) && QLA_DEBUG_DELAY
// Test build only (the forced-delay library): qla_test_fail_launches(n) makes
// the next n launches report a runtime rejection, so that the QLA_ERR_LAUNCH
// path of every entry point can be exercised without a failing launch.
std::atomic<int> g_fail_launches{0};
bool injected_failure()
{
    int n = g_fail_launches.load();
    while (n > 0 && !g_fail_launches.compare_exchange_weak(n, n - 1)) {
    }
    return n > 0;
}
#else
constexpr bool injected_failure() { return false; }
#endif

}  // namespace

extern "C" {

#if defined(QLA_DEBUG_DELAY) && QLA_DEBUG_DELAY
QLA_API int qla_test_fail_launches(int n)
{
    g_fail_launches.store(n > 0 ? n : 0);
    return QLA_OK;
}
// 1 if a plain call of this shape (chains of n_seg segments) runs two tiles
// per workgroup on a device with `cus` compute units, else 0.
QLA_API int qla_test_pairs_tiles(int K, long long chains, int V, int n_seg, int cus)
{
    return qla::plain_call_pairs_tiles(K, chains, V, n_seg, cus) ? 1 : 0;
}
#endif

int qla_correct_h0(const float* H, const float* M, const float* S0, float* out, int layout, int direction,
                   int batch, int heads, int n_seg, int K, int V, void* stream)
{
    if (!valid_layout(layout) || !valid_direction(direction)) return QLA_ERR_ENUM;
    int rc = check_shape(batch, heads, n_seg, K, V);
    if (rc != QLA_OK) return rc;
    const long long chains = (long long)batch * heads;
    if (chains == 0 || n_seg == 0) return QLA_OK;
    if ((rc = check_buffers(H, M, S0, out, chains, chains * n_seg, K, V)) != QLA_OK) return rc;

    qla::LaunchArgs a{H, M, S0, out, layout, direction, chains, heads, n_seg, K, V, stream, device_cus()};
    if (injected_failure()) return QLA_ERR_LAUNCH;
    clear_stale_error();
    return qla::launch_correct_h0(a) == hipSuccess ? QLA_OK : QLA_ERR_LAUNCH;
}

int qla_correct_h0_grouped(const float* H, const float* M, const float* S0, float* out,
                           const qla_head_group* groups, int n_groups, int batch, int heads, int n_seg, int K,
                           int V, void* stream)
{
    if (!groups || n_groups < 1 || n_groups > QLA_MAX_GROUPS) return QLA_ERR_GROUPS;
    for (int i = 0; i < n_groups; ++i)
        if (!valid_layout(groups[i].layout) || !valid_direction(groups[i].direction)) return QLA_ERR_ENUM;
    int rc = check_shape(batch, heads, n_seg, K, V);
    if (rc != QLA_OK) return rc;

    // The groups must partition [0, heads): each in range, pairwise disjoint,
    // and their sizes add up to heads.
    long long covered = 0;
    qla::GroupTable table{};
    table.n = n_groups;
    for (int i = 0; i < n_groups; ++i) {
        const qla_head_group& gi = groups[i];
        if (gi.head_count < 1 || gi.head_begin < 0 || (long long)gi.head_begin + gi.head_count > heads)
            return QLA_ERR_GROUPS;
        for (int k = 0; k < i; ++k) {
            const qla_head_group& gk = groups[k];
            if (gi.head_begin < gk.head_begin + gk.head_count && gk.head_begin < gi.head_begin + gi.head_count)
                return QLA_ERR_GROUPS;
        }
        covered += gi.head_count;
        table.begin[i] = gi.head_begin;
        table.count[i] = gi.head_count;
        table.variant[i] = 2 * gi.layout + gi.direction;
    }
    if (covered != heads) return QLA_ERR_GROUPS;

    const long long chains = (long long)batch * heads;
    if (chains == 0 || n_seg == 0) return QLA_OK;
    if ((rc = check_buffers(H, M, S0, out, chains, chains * n_seg, K, V)) != QLA_OK) return rc;

    qla::LaunchArgs a{H, M, S0, out, -1, -1, chains, heads, n_seg, K, V, stream, device_cus()};
    if (injected_failure()) return QLA_ERR_LAUNCH;
    clear_stale_error();
    return qla::launch_correct_h0_grouped(a, table) == hipSuccess ? QLA_OK : QLA_ERR_LAUNCH;
}

int qla_correct_h0_varlen(const float* H, const float* M, const float* S0, float* out, int layout, int direction,
                          const int* seg_offsets, int n_seqs, int heads, int K, int V, void* stream)
{
    if (!valid_layout(layout) || !valid_direction(direction)) return QLA_ERR_ENUM;
    if (!seg_offsets || n_seqs < 0 || n_seqs > QLA_MAX_SEQS || seg_offsets[0] != 0) return QLA_ERR_SEQS;
    qla::SeqTable seqs{};
    seqs.n = n_seqs;
    seqs.offs[0] = 0;
    for (int b = 0; b < n_seqs; ++b) {
        if (seg_offsets[b + 1] < seg_offsets[b]) return QLA_ERR_SEQS;
        seqs.offs[b + 1] = seg_offsets[b + 1];
    }
    int rc = check_shape(n_seqs, heads, 0, K, V);
    if (rc != QLA_OK) return rc;
    const long long chains = (long long)n_seqs * heads;
    const long long segments = (long long)heads * seg_offsets[n_seqs];
    // Segment offsets inside the kernel are int: heads * offset must fit.
    if ((long long)heads * seg_offsets[n_seqs] > INT32_MAX) return QLA_ERR_SHAPE;
    if (chains == 0 || segments == 0) return QLA_OK;
    if ((rc = check_buffers(H, M, S0, out, chains, segments, K, V)) != QLA_OK) return rc;

    qla::LaunchArgs a{H, M, S0, out, layout, direction, chains, heads, -1, K, V, stream, device_cus()};
    if (injected_failure()) return QLA_ERR_LAUNCH;
    clear_stale_error();
    return qla::launch_correct_h0_varlen(a, seqs) == hipSuccess ? QLA_OK : QLA_ERR_LAUNCH;
}

const char* qla_status_str(int status)
{
    switch (status) {
    case QLA_OK: return "ok";
    case QLA_ERR_NULL: return "H, M or out is NULL";
    case QLA_ERR_ENUM: return "layout or direction is not a known value";
    case QLA_ERR_SHAPE: return "unsupported shape (K must be a multiple of 16 in [16, 256]; V a multiple of 4 in "
                               "[4, 4096]; counts >= 0; grid within the launch limits)";
    case QLA_ERR_ALIGN: return "a buffer is not 16-byte aligned";
    case QLA_ERR_ALIAS: return "out overlaps H (other than exactly in place), M or S0";
    case QLA_ERR_GROUPS: return "head groups do not partition [0, heads) (or too many groups)";
    case QLA_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
    case QLA_ERR_MEMORY: return "a buffer is not device memory or is smaller than the call needs";
    case QLA_ERR_SEQS: return "segment offsets are NULL, not starting at 0, decreasing, or for more than "
                              "QLA_MAX_SEQS sequences";
    default: return "unknown status";
    }
}

}  // extern "C"
