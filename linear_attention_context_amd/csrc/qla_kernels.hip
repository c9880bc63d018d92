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

#ifndef QLA_LDS_PAD
#define QLA_LDS_PAD 8
#endif
#ifndef QLA_MLOAD_AUX
#define QLA_MLOAD_AUX 0
#endif
#ifndef QLA_HLOAD_AUX
#define QLA_HLOAD_AUX 0
#endif
#ifndef QLA_STORE_AUX
#define QLA_STORE_AUX 2  // non-temporal: out is not re-read
#endif
#ifndef QLA_BARRIER_FIRST
#define QLA_BARRIER_FIRST 0
#endif
constexpr int kTileV = 16;  // kv-view columns per workgroup

// Waves per workgroup.  Forward at K >= 128 runs two waves per SIMD, so one
// wave's operand waits are covered by the other's MFMAs.  Backward keeps
// four: its M share is a column block, and 32 columns per wave make each
// load a whole 128-byte line per row (16 columns would halve that).  The
// grouped kernel has one block size for all its groups and uses eight.
#ifndef QLA_WAVES
#define QLA_WAVES(K, FWD) ((K) >= 128 && (FWD) ? 8 : 4)
#endif
#ifndef QLA_GROUPED_WAVES
#define QLA_GROUPED_WAVES(K) ((K) >= 128 ? 8 : 4)
#endif
// Prefetch distance in units (panels) of M.
#ifndef QLA_PREFETCH_UNITS
#define QLA_PREFETCH_UNITS(K, FWD) ((K) >= 256 ? 1 : (K) >= 128 ? ((FWD) ? 3 : 2) : 3)
#endif

template <int K, int WAVES_, bool FWD_>
struct Shape {
    static constexpr int WAVES = WAVES_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int ROWS = K / WAVES;        // output rows per wave
    static constexpr int T = ROWS / 16;           // 16-row MFMA tiles per wave
    static constexpr int KP = K >= 256 ? 64 : K;  // k-width of one M panel
    static constexpr int NP = K / KP;             // panels per step
    static constexpr int BP = KP / 16;            // 16-wide k blocks per panel
    static constexpr int LS = K + QLA_LDS_PAD;    // LDS row stride (floats)
    static constexpr int STATE_FLOATS = 2 * kTileV * LS;  // two state slots
    static constexpr int STAGE_FLOATS = ROWS * KP;          // one wave's M panel share
    // Forward staging slots per wave: two (the next panel is written while
    // this one is read) when they fit in the 160 KiB of LDS, else one.
    static constexpr int SS =
        (STATE_FLOATS + WAVES * 2 * STAGE_FLOATS) * 4 <= 160 * 1024 && QLA_PREFETCH_UNITS(K, FWD_) >= 2 ? 2 : 1;
    static constexpr int RPI = 256 / KP;                    // M rows per coalesced load instruction
    // Prefetch distance in panels (see Tile::prefetch).
    static constexpr int D = QLA_PREFETCH_UNITS(K, FWD_);
    static_assert(ROWS % 16 == 0, "K must be a multiple of 64");
    static_assert(NP <= 4, "at most four panels per step");
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
template <int AUX = 0>
__device__ __forceinline__ f4 bload4(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ f2 bload2(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(f2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, AUX));
}
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, unsigned off, f4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, (int)off, 0, QLA_STORE_AUX);
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

template <int K, int LAYOUT, int DIR, int WAVES>
struct Tile {
    using S = Shape<K, WAVES, DIR == QLA_DIR_FWD>;
    static constexpr int T = S::T, KP = S::KP, NP = S::NP, BP = S::BP, LS = S::LS;
    static constexpr bool KV = LAYOUT == QLA_LAYOUT_KV;
    static constexpr bool FWD = DIR == QLA_DIR_FWD;
    static constexpr unsigned kMatBytes = (unsigned)K * K * 4u;
    // LDS: two state slots, plus one M staging slot per wave when forward.
    static constexpr int SS = S::SS;
    static constexpr int SF = S::STAGE_FLOATS;
    static constexpr int LDS_FLOATS = S::STATE_FLOATS + (FWD ? S::WAVES * SS * SF : 0);

    // Per-lane constants of one workgroup.
    struct Lane {
        int wave, g, c, a0;
        unsigned hoff[T];  // byte offsets of the lane's H/out vectors (kOutOfRange if masked)
        unsigned moff;     // byte offset of the lane's first M operand (backward)
        unsigned mcoal;    // byte offset of the lane's first coalesced M chunk (forward)
        int prot, brot;    // k-order rotation of this wave: panels, then 16-k blocks in a panel
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
        L.moff = 4u * (unsigned)(4 * L.g * K + L.a0 + T * L.c);
        // Each wave walks the k range starting at its own rows (k = a0 ...):
        // the state of those rows is its own output, readable before the
        // other waves have written theirs.
        L.prot = (L.wave * S::ROWS / KP) % NP;
        L.brot = (L.wave * S::ROWS / 16) % BP;
        L.mcoal = 4u * (unsigned)((L.a0 + lane / (KP / 4)) * K + 4 * (lane % (KP / 4)));
        return L;
    }

    static __device__ __forceinline__ void load_state(f4 (&h)[T], __amdgpu_buffer_rsrc_t r, const Lane& L)
    {
#pragma unroll
        for (int i = 0; i < T; ++i) h[i] = bload4(r, L.hoff[i]);
    }

    // Forward M staging.  Each wave owns a private LDS slot of ROWS x KP
    // floats, laid out [row][16-byte chunk] with the chunk index XORed by
    // (row & 15) so that both the line-wise writes and the MFMA-layout reads
    // (16 rows, same chunk) spread over all banks.  The slot is private to
    // the wave and LDS executes one wave's accesses in order, so the next
    // panel's writes cannot overtake this panel's reads: no barrier needed.
    static __device__ __forceinline__ int stage_off(int row, int chunk) { return row * KP + 4 * (chunk ^ (row & 15)); }

    // MFMA operand (a, k) = M[a0 + 16t + c][p*KP + 16b + 4g + q] for one (t, b).
    static __device__ __forceinline__ f4 stage_read(const float* stage, int t, int b, const Lane& L)
    {
        return *reinterpret_cast<const f4*>(stage + stage_off(16 * t + L.c, 4 * ((b + L.brot) & (BP - 1)) + L.g));
    }

    // Position of k block (panel p, block b of the wave's walk) in the k range.
    static __device__ __forceinline__ int panel_of(int p, const Lane& L) { return (p + L.prot) & (NP - 1); }
    static __device__ __forceinline__ int kblock(int p, int b, const Lane& L)
    {
        return panel_of(p, L) * BP + ((b + L.brot) & (BP - 1));
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

    // Prefetch ring.  The M stream of a chain is a sequence of units (one
    // panel of one step, NP units per step).  Unit u lives in register slot
    // u % R and is loaded D = R - 1 units ahead of its use, into the slot the
    // previous unit just freed.  H_j rides along with the first unit of its
    // step, in slot (step % RH).  Step loops are unrolled by F so that every
    // slot index is a compile-time constant.
    static constexpr int D = S::D;
    static constexpr int R = D + 1;
    static constexpr int RH = (NP - 1 + D) / NP + 1;
    static constexpr int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }
    static constexpr int F0 = R / gcd(R, NP);
    static constexpr int F = F0 * RH / gcd(F0, RH);
    static_assert(F >= 1 && F <= 6, "unroll block must be 1..6 steps");
    static_assert(!(FWD && SS == 2) || D >= 2, "two-slot staging stages a unit loaded two units ahead");

    // ---- one load / staging-write instruction at a time -------------------
    // Loads of one M panel (this wave's share): forward, T*BP whole-line
    // instructions (instruction i covers rows i*RPI .. i*RPI + RPI - 1 of the
    // share); backward, 4*BP T-wide instructions (one per (b, q)).
    static constexpr int kPanelLoads = FWD ? T * BP : 4 * BP;

    template <int I>
    static __device__ __forceinline__ void load_m(f4 (&m)[T][BP], __amdgpu_buffer_rsrc_t Mr, int panel, const Lane& L)
    {
        const int pa = panel_of(panel, L);
        if constexpr (FWD) {
            m[I / BP][I % BP] = bload4<QLA_MLOAD_AUX>(Mr, L.mcoal + 4u * (unsigned)(I * S::RPI * K + pa * KP));
        } else {
            // operand (a, k) = M[k][a], a = a0 + T*c + t, k = 16*kblock + 4g + q
            constexpr int b = I / 4, q = I % 4;
            const unsigned off = L.moff + 4u * (unsigned)((pa * KP + 16 * ((b + L.brot) & (BP - 1)) + q) * K);
            if constexpr (T == 1) {
                m[0][b][q] = bload1<QLA_MLOAD_AUX>(Mr, off);
            } else if constexpr (T == 2) {
                const f2 x = bload2<QLA_MLOAD_AUX>(Mr, off);
                m[0][b][q] = x[0];
                m[1][b][q] = x[1];
            } else {
                const f4 x = bload4<QLA_MLOAD_AUX>(Mr, off);
#pragma unroll
                for (int t = 0; t < T; ++t) m[t][b][q] = x[t];
            }
        }
    }

    // Forward staging write of register group I = t*BP + b of a panel share.
    template <int I>
    static __device__ __forceinline__ void stage_write_one(float* stage, const f4 (&m)[T][BP])
    {
        const int lane = threadIdx.x & 63;
        const int row = I * S::RPI + lane / (KP / 4);
        st4(stage + stage_off(row, lane % (KP / 4)), m[I / BP][I % BP]);
    }

    // Prefetch target of one panel: the unit D ahead.
    struct Prefetch {
        __amdgpu_buffer_rsrc_t Mr, Hr;
        int panel;
    };

    // Issue prefetch loads [LO, HI) of the target unit: M instructions first,
    // then (on a step's first panel) the T vectors of H.
    template <int LO, int HI, int TLS, int TP>
    static __device__ __forceinline__ void issue_loads(const Prefetch& pf, f4 (&m)[R][T][BP], f4 (&h)[RH][T],
                                                       const Lane& L)
    {
        if constexpr (LO < HI) {
            if constexpr (LO < kPanelLoads)
                load_m<LO>(m[(TLS * NP + TP) % R], pf.Mr, pf.panel, L);
            else
                h[TLS % RH][LO - kPanelLoads] = bload4<QLA_HLOAD_AUX>(pf.Hr, L.hoff[LO - kPanelLoads]);
            issue_loads<LO + 1, HI, TLS, TP>(pf, m, h, L);
        }
    }

    template <int LO, int HI>
    static __device__ __forceinline__ void issue_writes(float* stage, const f4 (&m)[T][BP])
    {
        if constexpr (LO < HI) {
            stage_write_one<LO>(stage, m);
            issue_writes<LO + 1, HI>(stage, m);
        }
    }

    // State operand of (panel P, block b): P[k][c], k = 16*kblock + 4g + q.
    template <int P, int LO, int HI>
    static __device__ __forceinline__ void read_pv(f4 (&pv)[K / 16], const float* cur, const Lane& L)
    {
        if constexpr (LO < HI) {
            pv[P * BP + LO] = *reinterpret_cast<const f4*>(cur + L.c * LS + 16 * kblock(P, LO, L) + 4 * L.g);
            read_pv<P, LO + 1, HI>(pv, cur, L);
        }
    }

    // Working set of one step.
    struct StepCtx {
        f4 acc[T];
        f4 pv[K / 16];
        f4 mo[3][T];  // forward: staged M operand, read two blocks ahead
        const float* cur;
        const float* st_cur;
        float* st_next;
    };

    // Blocks of a step, in the wave's k order: the first T blocks are the
    // wave's own rows, whose state the wave wrote itself; the barrier that
    // publishes the other waves' rows sits after the first of them, so its
    // wait and the following state reads overlap the remaining own-row MFMAs.
    static constexpr int kOwn = T;  // 16-k blocks of own rows
    static constexpr int kOwnP0 = kOwn < BP ? kOwn : BP;

    // One 16-k block B of panel P (local step LSX): half the block's MFMAs,
    // staged reads two blocks ahead, this block's share of the prefetch loads
    // and of the next panel's staging writes, the other half of the MFMAs.
    // Each block is its own scheduling region so the CU's vector-memory and
    // LDS work is spread through the matrix-core work.
    template <int LSX, int P, int B>
    static __device__ __forceinline__ void block(StepCtx& X, const Prefetch& pf, f4 (&m)[R][T][BP],
                                                 f4 (&h)[RH][T], const Lane& L)
    {
        constexpr int slot = (LSX * NP + P) % R;
        constexpr int TLS = LSX + (P + D) / NP, TP = (P + D) % NP;
        constexpr int NL = kPanelLoads + (TP == 0 ? T : 0);
        constexpr int l0 = NL * B / BP, l1 = NL * (B + 1) / BP;
        constexpr int NW = (FWD && SS == 2) ? T * BP : 0;
        constexpr int w0 = NW * B / BP, w1 = NW * (B + 1) / BP;
        constexpr int nr = (FWD && B + 2 < BP) ? T : 0;

        auto mfma = [&](int q) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const float pk = X.pv[P * BP + B][q];
                const float mk = FWD ? X.mo[B % 3][t][q] : m[slot][t][B][q];
                if (KV)
                    X.acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(pk, mk, X.acc[t], 0, 0, 0);
                else
                    X.acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(mk, pk, X.acc[t], 0, 0, 0);
            }
        };
        mfma(0);
        mfma(1);
        if constexpr (nr > 0) {
#pragma unroll
            for (int t = 0; t < T; ++t) X.mo[(B + 2) % 3][t] = stage_read(X.st_cur, t, B + 2, L);
        }
        issue_loads<l0, l1, TLS, TP>(pf, m, h, L);
        if constexpr (NW > 0) issue_writes<w0, w1>(X.st_next, m[(LSX * NP + P + 1) % R]);
        mfma(2);
        mfma(3);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * T, 0);                                // MFMA
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);             // DS read
        if constexpr (l1 > l0) __builtin_amdgcn_sched_group_barrier(0x020, l1 - l0, 0);       // VMEM read
        if constexpr (w1 > w0) __builtin_amdgcn_sched_group_barrier(0x200, w1 - w0, 0);       // DS write
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * T, 0);                                // MFMA
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (P == 0 && B == 0 && !QLA_BARRIER_FIRST) {
            // Publish / acquire the state rows of the other waves, then read
            // their part of this panel's state operand.
            lds_handoff();
            read_pv<0, kOwnP0, BP>(X.pv, X.cur, L);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (B + 1 < BP) block<LSX, P, B + 1>(X, pf, m, h, L);
    }

    // Panel P of step s (local index LSX).
    template <int LSX, int P>
    static __device__ __forceinline__ void panel(int s, StepCtx& X, const Chain& C, f4 (&m)[R][T][BP],
                                                 f4 (&h)[RH][T], float* stage, const Lane& L)
    {
        constexpr int slot = (LSX * NP + P) % R;
        // Prefetch target: the unit D ahead, or an empty resource past the chain's end.
        const int ts = s + (P + D) / NP;
        const bool live = ts < C.n_seg;
        const int tj = live ? seg(C, ts) : 0;
        const Prefetch pf{rsrc(C.M + (size_t)tj * K * K, live ? kMatBytes : 0u),
                          rsrc(C.H + (size_t)tj * (L.state_bytes / 4), live ? L.state_bytes : 0u), (P + D) % NP};
        // Forward: this panel's M is read from staging slot (unit & 1),
        // written during the previous panel (two slots) or just below (one).
        // The next panel goes into the other slot, which the previous panel
        // last read: this wave issued those reads before these writes, and LDS
        // runs one wave's accesses in order.
        const int unit = s * NP + P;
        X.st_cur = stage + (SS == 2 ? (unit & 1) * SF : 0);
        X.st_next = stage + (SS == 2 ? ((unit + 1) & 1) * SF : 0);

        // State operand: panel 0's own-row blocks (own writes, no barrier
        // needed); later panels after the barrier, in full.
        if constexpr (P == 0) read_pv<0, 0, kOwnP0>(X.pv, X.cur, L);
        else read_pv<P, 0, BP>(X.pv, X.cur, L);
        if constexpr (FWD && SS == 1) issue_writes<0, T * BP>(stage, m[slot]);
        if constexpr (FWD) {
#pragma unroll
            for (int t = 0; t < T; ++t) X.mo[0][t] = stage_read(X.st_cur, t, 0, L);
            if constexpr (BP > 1) {
#pragma unroll
                for (int t = 0; t < T; ++t) X.mo[1][t] = stage_read(X.st_cur, t, 1, L);
            }
        }
        if constexpr (P == 0 && QLA_BARRIER_FIRST) {
            lds_handoff();
            read_pv<0, kOwnP0, BP>(X.pv, X.cur, L);
        }
        __builtin_amdgcn_sched_barrier(0);
        block<LSX, P, 0>(X, pf, m, h, L);
        if constexpr (P + 1 < NP) panel<LSX, P + 1>(s, X, C, m, h, stage, L);
    }

    // One segment step with compile-time local index LSX (position in the
    // unrolled block).  Reads LDS state slot s & 1, writes slot (s + 1) & 1.
    // Slot (s+1)&1 was last read during step s-1; every wave finished those
    // reads before arriving at the barrier inside step s, and the writes come
    // after it.  The other waves' rows of slot s&1 are read after that same
    // barrier, which no wave reaches before its step s-1 writes landed.
    template <int LSX>
    static __device__ __forceinline__ void step(int s, const Chain& C, f4 (&m)[R][T][BP], f4 (&h)[RH][T],
                                                float* lds, const Lane& L)
    {
        const int j = seg(C, s);
        float* nxt = lds + ((s + 1) & 1) * (kTileV * LS);
        float* stage = lds + S::STATE_FLOATS + L.wave * SS * SF;

        __builtin_amdgcn_sched_barrier(0);
        debug_delay(L.wave, s, 0);
        StepCtx X;
        X.cur = lds + (s & 1) * (kTileV * LS);
#pragma unroll
        for (int t = 0; t < T; ++t) X.acc[t] = f4{0.f, 0.f, 0.f, 0.f};
        panel<LSX, 0>(s, X, C, m, h, stage, L);

        // Correct: P = Y + X(H_j); emit out_j; hand the state to the next step.
        f4 hx[T];
        frag_from_vecs(hx, h[LSX % RH]);
#pragma unroll
        for (int t = 0; t < T; ++t) X.acc[t] += hx[t];
        f4 ov[T];
        vecs_from_frag(ov, X.acc);
        const __amdgpu_buffer_rsrc_t Or = rsrc(C.out + (size_t)j * (L.state_bytes / 4), L.state_bytes);
#pragma unroll
        for (int i = 0; i < T; ++i) bstore4(Or, L.hoff[i], ov[i]);
        debug_delay(L.wave, s, 1);
        put_state(nxt, X.acc, L);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Remaining steps after the unrolled loop (fewer than F), straight-line.
    template <int LSX>
    static __device__ __forceinline__ void tail(int s, int rem, const Chain& C, f4 (&m)[R][T][BP],
                                                f4 (&h)[RH][T], float* lds, const Lane& L)
    {
        if constexpr (LSX < F - 1) {
            if (rem > LSX) {
                step<LSX>(s + LSX, C, m, h, lds, L);
                tail<LSX + 1>(s, rem, C, m, h, lds, L);
            }
        }
    }

    // Prologue loads: units 0 .. D-1 (and the H of the steps they start).
    template <int V_>
    static __device__ __forceinline__ void prologue(const Chain& C, f4 (&m)[R][T][BP], f4 (&h)[RH][T],
                                                    const Lane& L)
    {
        if constexpr (V_ < D) {
            constexpr int TLS = V_ / NP, TP = V_ % NP;
            const bool live = TLS < C.n_seg;
            const int tj = live ? seg(C, TLS) : 0;
            const Prefetch pf{rsrc(C.M + (size_t)tj * K * K, live ? kMatBytes : 0u),
                              rsrc(C.H + (size_t)tj * (L.state_bytes / 4), live ? L.state_bytes : 0u), TP};
            issue_loads<0, kPanelLoads + (TP == 0 ? T : 0), TLS, TP>(pf, m, h, L);
            prologue<V_ + 1>(C, m, h, L);
        }
    }

    static __device__ __forceinline__ void run(const float* H, const float* M, const float* S0, float* out,
                                               int n_seg, int V, size_t chain, int tile, float* lds)
    {
        const Lane L = make_lane(tile * kTileV, V);
        const size_t state = (size_t)K * V;
        const Chain C{M + chain * (size_t)n_seg * K * K, H + chain * state * n_seg, out + chain * state * n_seg,
                      n_seg};

        f4 m[R][T][BP];
        f4 h[RH][T];
        // Prologue: the first D units of M (and their steps' H), then the
        // initial state into LDS slot 0.
        prologue<0>(C, m, h, L);
        if constexpr (FWD && SS == 2) issue_writes<0, T * BP>(lds + S::STATE_FLOATS + L.wave * SS * SF, m[0]);
        {
            f4 sv[T], sx[T];
            load_state(sv, rsrc(S0 ? S0 + chain * state : H, S0 ? L.state_bytes : 0u), L);
            frag_from_vecs(sx, sv);
            put_state(lds, sx, L);
        }

        int s = 0;
        for (; s + F <= n_seg; s += F) {
            step<0>(s, C, m, h, lds, L);
            if constexpr (F > 1) step<1 % F>(s + 1, C, m, h, lds, L);
            if constexpr (F > 2) step<2 % F>(s + 2, C, m, h, lds, L);
            if constexpr (F > 3) step<3 % F>(s + 3, C, m, h, lds, L);
            if constexpr (F > 4) step<4 % F>(s + 4, C, m, h, lds, L);
            if constexpr (F > 5) step<5 % F>(s + 5, C, m, h, lds, L);
        }
        tail<0>(s, n_seg - s, C, m, h, lds, L);
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
struct Plain {
    static constexpr int WAVES = QLA_WAVES(K, DIR == QLA_DIR_FWD);
    using Tl = Tile<K, LAYOUT, DIR, WAVES>;
};

template <int K, int LAYOUT, int DIR>
__global__ __launch_bounds__(64 * QLA_WAVES(K, DIR == QLA_DIR_FWD)) void correct_h0_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int n_seg, int V, int tiles)
{
    using Tl = typename Plain<K, LAYOUT, DIR>::Tl;
    __shared__ __attribute__((aligned(16))) float lds[Tl::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    Tl::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds);
}

template <int K>
__global__ __launch_bounds__(64 * QLA_GROUPED_WAVES(K)) void correct_h0_grouped_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int n_seg, int V, int tiles, int heads,
    GroupTable table)
{
    constexpr int W = QLA_GROUPED_WAVES(K);
    constexpr int F1 = Tile<K, QLA_LAYOUT_KV, QLA_DIR_FWD, W>::LDS_FLOATS;
    constexpr int F2 = Tile<K, QLA_LAYOUT_KV, QLA_DIR_BWD, W>::LDS_FLOATS;
    __shared__ __attribute__((aligned(16))) float lds[F1 > F2 ? F1 : F2];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    const int head = chain % heads;
    int variant = 0;
    for (int i = 0; i < table.n; ++i)
        if (head >= table.begin[i] && head < table.begin[i] + table.count[i]) variant = table.variant[i];
    switch (variant) {
    case 0: Tile<K, QLA_LAYOUT_KV, QLA_DIR_FWD, W>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    case 1: Tile<K, QLA_LAYOUT_KV, QLA_DIR_BWD, W>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    case 2: Tile<K, QLA_LAYOUT_VK, QLA_DIR_FWD, W>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    default: Tile<K, QLA_LAYOUT_VK, QLA_DIR_BWD, W>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    }
}

template <int K, int LAYOUT, int DIR>
hipError_t launch_one(const LaunchArgs& a)
{
    const int tiles = (a.V + kTileV - 1) / kTileV;
    const dim3 grid((unsigned)(a.chains * tiles));
    hipLaunchKernelGGL((correct_h0_kernel<K, LAYOUT, DIR>), grid, dim3(64 * Plain<K, LAYOUT, DIR>::WAVES), 0,
                       (hipStream_t)a.stream, a.H,
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
    hipLaunchKernelGGL((correct_h0_grouped_kernel<K>), grid, dim3(64 * QLA_GROUPED_WAVES(K)), 0, (hipStream_t)a.stream,
                       a.H, a.M,
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
