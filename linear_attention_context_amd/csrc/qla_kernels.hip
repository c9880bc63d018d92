// qla_kernels.hip -- gfx950 kernels for the context-parallel state-correction
// recurrence (Antarx Memos, FlashQLA correction note: "一次 TileLang Warp
// Specialization 数值错误的定位与修复：从双缓冲竞争到 membar").
//
// What is computed (section "理解三个缓冲区，才能判断哪里需要同步": local
// states H_j, propagation matrices M_j, the corrected state is the previous
// one propagated through M_j plus H_j; section "从版本升级后的数值偏差开始":
// forward initial-state and backward terminal-state correction, kv / vk
// layouts).  In the kv view X (X = S for kv, X = S^T for vk):
//     forward : P <- M_j   P + X(H_j), j ascending,  out_j = P
//     backward: P <- M_j^T P + X(H_j), j descending, out_j = P
//
// Work decomposition.  Each column of the kv view evolves on its own
// (p <- M_j p + h_j), so one workgroup carries one chain's recurrence for a
// 16-column tile of the state, serially over the segments, and the chains x
// tiles fill the GPU.  The workgroup's four waves split the K output rows: wave
// w computes rows [w*K/4, (w+1)*K/4).  A wave therefore needs only its own
// quarter of every M_j (its rows forward, its columns backward) and of every
// H_j, and nothing it loads from HBM is shared with another wave: those
// operands go straight from global memory into the wave's registers, one
// panel ahead of use (a panel is a 64 KiB slice of M for the workgroup), in a
// two-slot register ring.  The pages' Hopper kernel staged H and M through
// shared-memory slots filled by a separate producer; here the prefetch target
// is private to the consuming wave, so the slot-reuse race the note diagnoses
// (section "决定性证据：错误值来自同一槽位的下一代": a slot read after it was
// refilled with the segment two steps away) has no shared slot to happen in.
//
// The one shared buffer is the state exchange (the note's hd_shared role): each
// step every wave needs all K rows of the previous state for its MFMA operand.
// It lives in LDS as two slots.  Step s reads slot s&1 and writes slot (s+1)&1,
// then every wave waits for its own LDS traffic (lgkmcnt(0)) and meets the
// others at one s_barrier.  The slot written at step s was last read at step
// s-1; every wave finished those reads before it arrived at the barrier that
// closes step s-1, and no wave writes before passing that barrier.  The reads
// of step s+1 come after the barrier that closes step s, which no wave reaches
// before its writes landed.  Read-before-reuse holds by construction.
//
// Matrix cores: v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate).  Lane l =
// 16*g + c feeds operand value (row c, k = 4g + q) on the q-th of four
// instructions; the contraction order inside a 16-wide k block is thereby
// {4g+q}, fixed, so results are bit-reproducible.  The accumulator fragment
// (lane l, register r) is element (4g + r, c) of the 16x16 tile.  For kv the
// tile computed is Y^T (rows = state columns v), for vk it is Y (rows = state
// rows a): in both cases a lane's four registers are four consecutive floats
// of the stored matrix, so H loads and out stores are 128-bit.
#include <hip/hip_runtime.h>

#include "qla_internal.h"

namespace qla {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileV = 16;  // kv-view columns per workgroup

template <int K>
struct Shape {
    static constexpr int ROWS = K / kWaves;       // output rows per wave
    static constexpr int T = ROWS / 16;           // 16-row MFMA tiles per wave
    static constexpr int KP = K >= 256 ? 64 : K;  // k-width of one M panel
    static constexpr int NP = K / KP;             // panels per step
    static constexpr int BP = KP / 16;            // 16-wide k blocks per panel
    static constexpr int LS = K + 4;              // LDS row stride (floats)
    static constexpr int LDS_FLOATS = 2 * kTileV * LS;
    static_assert(ROWS % 16 == 0, "K must be a multiple of 64");
    static_assert(NP == 1 || NP % 2 == 0, "panel ring needs NP = 1 or even");
};

// Wait until this wave's LDS accesses are done, then meet the other waves.
// The asm's memory clobber keeps the compiler from moving any memory access
// across it; global loads in flight (the prefetch) are deliberately not waited.
__device__ __forceinline__ void lds_handoff()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Buffer resources.  All H/M/S0/out traffic goes through raw buffer
// instructions: a lane whose byte offset is past num_records reads zeros and
// its store is dropped by the hardware, and a resource with num_records = 0
// turns a whole prefetch into a no-op.  That keeps the steady-state loop free
// of branches around memory operations, so the compiler's wait counting sees
// one straight-line pattern and waits only for the data each MFMA needs.
constexpr int kRsrcWord3 = 0x00020000;        // raw 32-bit buffer, gfx9 family
constexpr unsigned kOutOfRange = 0x80000000u;  // byte offset beyond any resource

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const float* base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ f4 bload4(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ f2 bload2(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(f2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, unsigned off, f4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void st4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }
__device__ __forceinline__ void st2(float* p, f2 v) { *reinterpret_cast<f2*>(p) = v; }

// Optional forced-delay schedule (built only into the race-test library): one
// wave per step sleeps before reading the shared state slot, another before
// writing the next one.  Results must not change.
__device__ __forceinline__ void debug_delay(int wave, int s, int which)
{
#if defined(QLA_DEBUG_DELAY) && QLA_DEBUG_DELAY
    if (wave == ((s + which) & 3)) {
        __builtin_amdgcn_s_sleep(100);
        __builtin_amdgcn_s_sleep(100);
    }
#else
    (void)wave;
    (void)s;
    (void)which;
#endif
}

template <int K, int LAYOUT, int DIR>
struct Tile {
    using S = Shape<K>;
    static constexpr int T = S::T, KP = S::KP, NP = S::NP, BP = S::BP, LS = S::LS;
    static constexpr bool KV = LAYOUT == QLA_LAYOUT_KV;
    static constexpr bool FWD = DIR == QLA_DIR_FWD;
    static constexpr unsigned kMatBytes = (unsigned)K * K * 4u;

    // Per-lane constants of one workgroup.
    struct Lane {
        int wave, g, c, a0;
        unsigned hoff[T];  // byte offsets of the lane's H/out vectors (kOutOfRange if masked)
        unsigned moff;     // byte offset of the lane's first M operand
        unsigned state_bytes;
    };

    // Row of the kv view held by fragment row i of tile t: tiles are
    // contiguous 16-row blocks forward; backward they interleave with stride
    // T so that a lane's T values of one M row are adjacent in memory.
    static __device__ __forceinline__ int arow(int a0, int t, int i)
    {
        return FWD ? a0 + 16 * t + i : a0 + T * i + t;
    }

    // Fragment element (t, r) of the state <-> component of the lane's
    // 16-byte H/out vectors.  kv and vk-forward: vector t, component r.
    // vk-backward: the lane's 4T values are contiguous, element (t, r) at
    // flat index T*r + t.
    static constexpr int vec_of(int t, int r) { return (KV || FWD) ? t : (T * r + t) >> 2; }
    static constexpr int comp_of(int t, int r) { return (KV || FWD) ? r : (T * r + t) & 3; }

    static __device__ __forceinline__ Lane make_lane(int v0, int V)
    {
        Lane L;
        const int lane = threadIdx.x & 63;
        L.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        L.g = lane >> 4;
        L.c = lane & 15;
        L.a0 = L.wave * S::ROWS;
        L.state_bytes = (unsigned)K * V * 4u;
        const bool valid = KV ? (v0 + 4 * L.g < V) : (v0 + L.c < V);
#pragma unroll
        for (int i = 0; i < T; ++i) {
            int e;
            if (KV) e = arow(L.a0, i, L.c) * V + v0 + 4 * L.g;
            else if (FWD) e = (v0 + L.c) * K + L.a0 + 16 * i + 4 * L.g;
            else e = (v0 + L.c) * K + L.a0 + 4 * T * L.g + 4 * i;
            L.hoff[i] = valid ? 4u * (unsigned)e : kOutOfRange;
        }
        // Forward: M[a0 + c][4g]; backward: M[4g][a0 + T*c] (panel/block/tile offsets added per load).
        L.moff = FWD ? 4u * (unsigned)((L.a0 + L.c) * K + 4 * L.g) : 4u * (unsigned)(4 * L.g * K + L.a0 + T * L.c);
        return L;
    }

    // Load panel p of one M matrix (this wave's share) into a ring slot.
    static __device__ __forceinline__ void load_panel(f4 (&m)[T][BP], __amdgpu_buffer_rsrc_t Mr, int p,
                                                      const Lane& L)
    {
        if (FWD) {
            // operand (a, k) = M[a][k], a = a0 + 16t + c, k = p*KP + 16b + 4g + q: 16 bytes per (t, b).
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int b = 0; b < BP; ++b)
                    m[t][b] = bload4(Mr, L.moff + 4u * (unsigned)(16 * t * K + p * KP + 16 * b));
        } else {
            // Backward uses M^T: operand (a, k) = M[k][a], a = a0 + T*c + t.  The
            // T tiles' values of one M row are adjacent: one T-wide load per (b, q).
#pragma unroll
            for (int b = 0; b < BP; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const unsigned off = L.moff + 4u * (unsigned)((p * KP + 16 * b + q) * K);
                    if (T == 1) {
                        m[0][b][q] = bload1(Mr, off);
                    } else if (T == 2) {
                        const f2 x = bload2(Mr, off);
                        m[0][b][q] = x[0];
                        m[T - 1][b][q] = x[1];
                    } else {
                        const f4 x = bload4(Mr, off);
#pragma unroll
                        for (int t = 0; t < T; ++t) m[t][b][q] = x[t & 3];
                    }
                }
        }
    }

    static __device__ __forceinline__ void load_state(f4 (&h)[T], __amdgpu_buffer_rsrc_t r, const Lane& L)
    {
#pragma unroll
        for (int i = 0; i < T; ++i) h[i] = bload4(r, L.hoff[i]);
    }

    // Write the lane's fragment of the state into one LDS slot ([v][k] order).
    static __device__ __forceinline__ void put_state(float* buf, const f4 (&x)[T], const Lane& L)
    {
        const int g = L.g, c = L.c, a0 = L.a0;
        if (KV) {
            // element (t, r): column v = 4g + r, row a = arow(t, c)
            if (FWD) {
#pragma unroll
                for (int t = 0; t < T; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) buf[(4 * g + r) * LS + a0 + 16 * t + c] = x[t][r];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float* dst = buf + (4 * g + r) * LS + a0 + T * c;
                    if (T == 1) {
                        dst[0] = x[0][r];
                    } else if (T == 2) {
                        st2(dst, f2{x[0][r], x[T - 1][r]});
                    } else {
                        st4(dst, f4{x[0][r], x[1 % T][r], x[2 % T][r], x[3 % T][r]});
                    }
                }
            }
        } else {
            // element (t, r): column v = c, row a = arow(t, 4g + r)
            if (FWD) {
#pragma unroll
                for (int t = 0; t < T; ++t) st4(buf + c * LS + a0 + 16 * t + 4 * g, x[t]);
            } else {
                // rows a0 + 4Tg + (T r + t): the lane's 4T values are contiguous
#pragma unroll
                for (int i = 0; i < T; ++i) {
                    f4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int f = 4 * i + e;  // flat index = T*r + t
                        v[e] = x[f % T][f / T];
                    }
                    st4(buf + c * LS + a0 + 4 * T * g + 4 * i, v);
                }
            }
        }
    }

    static __device__ __forceinline__ void frag_from_vecs(f4 (&x)[T], const f4 (&h)[T])
    {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) x[t][r] = h[vec_of(t, r)][comp_of(t, r)];
    }

    static __device__ __forceinline__ void vecs_from_frag(f4 (&h)[T], const f4 (&x)[T])
    {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) h[vec_of(t, r)][comp_of(t, r)] = x[t][r];
    }

    struct Chain {
        const float* M;
        const float* H;
        float* out;
        int n_seg;
    };

    static __device__ __forceinline__ int seg(const Chain& C, int s) { return FWD ? s : C.n_seg - 1 - s; }

    // One segment step.  PAR = s & 1 selects the register ring slots and the
    // LDS state slot (read PAR, write PAR ^ 1).
    template <int PAR>
    static __device__ __forceinline__ void step(int s, const Chain& C, f4 (&m)[2][T][BP], f4 (&h)[2][T],
                                                float* lds, const Lane& L)
    {
        const int j = seg(C, s);
        const bool more = s + 1 < C.n_seg;
        const int jn = more ? seg(C, s + 1) : j;
        const float* cur = lds + PAR * (kTileV * LS);
        float* nxt = lds + (PAR ^ 1) * (kTileV * LS);
        const __amdgpu_buffer_rsrc_t Mr = rsrc(C.M + (size_t)j * K * K, kMatBytes);
        // Resources of the next step; empty after the last step, so its prefetch reads nothing.
        const __amdgpu_buffer_rsrc_t Mn = rsrc(C.M + (size_t)jn * K * K, more ? kMatBytes : 0u);
        const __amdgpu_buffer_rsrc_t Hn = rsrc(C.H + (size_t)jn * (L.state_bytes / 4), more ? L.state_bytes : 0u);

        f4 acc[T];
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};

        debug_delay(L.wave, s, 0);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int slot = (PAR * NP + p) & 1;
            // Prefetch the next panel (or the next step's first panel and H)
            // into the other ring slot before computing on this one.
            if (p + 1 < NP) {
                load_panel(m[slot ^ 1], Mr, p + 1, L);
            } else {
                load_panel(m[slot ^ 1], Mn, 0, L);
                load_state(h[PAR ^ 1], Hn, L);
            }
            // Keep the prefetch issued here, ahead of the MFMAs: left alone, the
            // scheduler sinks the loads below them to save registers, which
            // turns the prefetch into a stall at the next step.
            __builtin_amdgcn_sched_barrier(0);
            // Previous state, this panel's k range: P[k][c], k = p*KP + 16b + 4g + q.
            f4 pv[BP];
#pragma unroll
            for (int b = 0; b < BP; ++b)
                pv[b] = *reinterpret_cast<const f4*>(cur + L.c * LS + p * KP + 16 * b + 4 * L.g);
#pragma unroll
            for (int b = 0; b < BP; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        if (KV)
                            acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[b][q], m[slot][t][b][q], acc[t], 0, 0, 0);
                        else
                            acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(m[slot][t][b][q], pv[b][q], acc[t], 0, 0, 0);
                    }
        }

        // Correct: P = Y + X(H_j); emit out_j; hand the state to the next step.
        f4 hx[T];
        frag_from_vecs(hx, h[PAR]);
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t] += hx[t];
        f4 ov[T];
        vecs_from_frag(ov, acc);
        const __amdgpu_buffer_rsrc_t Or = rsrc(C.out + (size_t)j * (L.state_bytes / 4), L.state_bytes);
#pragma unroll
        for (int i = 0; i < T; ++i) bstore4(Or, L.hoff[i], ov[i]);
        debug_delay(L.wave, s, 1);
        put_state(nxt, acc, L);
        lds_handoff();
    }

    static __device__ __forceinline__ void run(const float* H, const float* M, const float* S0, float* out,
                                               int n_seg, int V, size_t chain, int tile, float* lds)
    {
        const Lane L = make_lane(tile * kTileV, V);
        const size_t state = (size_t)K * V;
        const Chain C{M + chain * (size_t)n_seg * K * K, H + chain * state * n_seg, out + chain * state * n_seg,
                      n_seg};

        f4 m[2][T][BP];
        f4 h[2][T];
        // Prologue: the first step's first panel and local state, then the
        // initial state into LDS slot 0.
        const int j0 = seg(C, 0);
        load_panel(m[0], rsrc(C.M + (size_t)j0 * K * K, kMatBytes), 0, L);
        load_state(h[0], rsrc(C.H + (size_t)j0 * state, L.state_bytes), L);
        {
            f4 sv[T], sx[T];
            load_state(sv, rsrc(S0 ? S0 + chain * state : H, S0 ? L.state_bytes : 0u), L);
            frag_from_vecs(sx, sv);
            put_state(lds, sx, L);
        }
        lds_handoff();

        int s = 0;
        for (; s + 1 < n_seg; s += 2) {
            step<0>(s, C, m, h, lds, L);
            step<1>(s + 1, C, m, h, lds, L);
        }
        if (s < n_seg) step<0>(s, C, m, h, lds, L);
    }
};

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  Renumber them so that consecutive logical ids -- the tiles of one
// chain, which all read the same M_j -- land on the same XCD and share its L2.
__device__ __forceinline__ int xcd_logical_id(int b, int G)
{
    const int q = G >> 3, r = G & 7, x = b & 7;
    const int base = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    return base + (b >> 3);
}

template <int K, int LAYOUT, int DIR>
__global__ __launch_bounds__(kThreads) void correct_h0_kernel(const float* H, const float* __restrict__ M,
                                                              const float* S0, float* out, int n_seg, int V,
                                                              int tiles)
{
    __shared__ __attribute__((aligned(16))) float lds[Shape<K>::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    Tile<K, LAYOUT, DIR>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds);
}

template <int K>
__global__ __launch_bounds__(kThreads) void correct_h0_grouped_kernel(const float* H, const float* __restrict__ M,
                                                                      const float* S0, float* out, int n_seg,
                                                                      int V, int tiles, int heads,
                                                                      GroupTable table)
{
    __shared__ __attribute__((aligned(16))) float lds[Shape<K>::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    const int head = chain % heads;
    int variant = 0;
    for (int i = 0; i < table.n; ++i)
        if (head >= table.begin[i] && head < table.begin[i] + table.count[i]) variant = table.variant[i];
    switch (variant) {
    case 0: Tile<K, QLA_LAYOUT_KV, QLA_DIR_FWD>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    case 1: Tile<K, QLA_LAYOUT_KV, QLA_DIR_BWD>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    case 2: Tile<K, QLA_LAYOUT_VK, QLA_DIR_FWD>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    default: Tile<K, QLA_LAYOUT_VK, QLA_DIR_BWD>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    }
}

template <int K, int LAYOUT, int DIR>
hipError_t launch_one(const LaunchArgs& a)
{
    const int tiles = (a.V + kTileV - 1) / kTileV;
    const dim3 grid((unsigned)(a.chains * tiles));
    hipLaunchKernelGGL((correct_h0_kernel<K, LAYOUT, DIR>), grid, dim3(kThreads), 0, (hipStream_t)a.stream, a.H,
                       a.M, a.S0, a.out, a.n_seg, a.V, tiles);
    return hipGetLastError();
}

template <int K>
hipError_t launch_k(const LaunchArgs& a)
{
    if (a.layout == QLA_LAYOUT_KV)
        return a.direction == QLA_DIR_FWD ? launch_one<K, QLA_LAYOUT_KV, QLA_DIR_FWD>(a)
                                          : launch_one<K, QLA_LAYOUT_KV, QLA_DIR_BWD>(a);
    return a.direction == QLA_DIR_FWD ? launch_one<K, QLA_LAYOUT_VK, QLA_DIR_FWD>(a)
                                      : launch_one<K, QLA_LAYOUT_VK, QLA_DIR_BWD>(a);
}

template <int K>
hipError_t launch_grouped_k(const LaunchArgs& a, const GroupTable& table)
{
    const int tiles = (a.V + kTileV - 1) / kTileV;
    const dim3 grid((unsigned)(a.chains * tiles));
    hipLaunchKernelGGL((correct_h0_grouped_kernel<K>), grid, dim3(kThreads), 0, (hipStream_t)a.stream, a.H, a.M,
                       a.S0, a.out, a.n_seg, a.V, tiles, a.heads, table);
    return hipGetLastError();
}

}  // namespace

int tiles_for(int V) { return (V + kTileV - 1) / kTileV; }

hipError_t launch_correct_h0(const LaunchArgs& a)
{
    switch (a.K) {
    case 64: return launch_k<64>(a);
    case 128: return launch_k<128>(a);
    case 256: return launch_k<256>(a);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_correct_h0_grouped(const LaunchArgs& a, const GroupTable& table)
{
    switch (a.K) {
    case 64: return launch_grouped_k<64>(a, table);
    case 128: return launch_grouped_k<128>(a, table);
    case 256: return launch_grouped_k<256>(a, table);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qla
