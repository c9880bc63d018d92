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
// tiles fill the GPU.  The workgroup's MFMA waves split the K output rows:
// wave w computes rows [w*K/W, (w+1)*K/W).
//
// The shared state (the note's hd_shared role): each step every wave needs
// all K rows of the previous state as its MFMA operand.  A wave's own rows it
// keeps in registers (its accumulator is laid out as the operand it feeds);
// the others come from LDS, which holds the state in two slots.  Step s opens
// with one barrier (each wave first waits for its own LDS traffic), reads the
// other waves' rows from slot s&1, and ends by writing its rows of the new
// state to slot (s+1)&1.  That slot was last read during step s-1, and every
// wave finished those reads before any wave passed the barrier that opens
// step s; the reads of step s+1 come after the barrier that opens it, which
// no wave reaches before its writes landed.  Read-before-reuse holds by
// construction.
//
// Staging of M.  At K <= 128 (DmaChain, both directions, also inside the
// grouped kernel), dedicated producer waves copy each M_j into one of two LDS
// stages, released by that same per-step barrier (the pages' Hopper kernel
// also had a producer, with its own two-slot buffers and hand-off; the
// slot-reuse race the note diagnoses, section
// "决定性证据：错误值来自同一槽位的下一代", a slot read after it was refilled with
// the segment two steps away, cannot happen here because a stage is refilled
// only after the barrier that every reader of its previous contents has
// passed), and warm later steps' lines into L2 right behind each copy.  At
// K = 256 (Tile) each wave prefetches exactly the share of M it consumes into
// a private register ring, forward through a private LDS slot.
//
// Matrix cores: v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate).  Lane l =
// 16*g + c feeds A(row c, k) and B(k, column c) with k = 4g + q on the q-th of
// four instructions; the contraction order inside a 16-wide k block is
// thereby fixed, so results are bit-reproducible.  The accumulator (lane l,
// register r) is element (4g + r, c) of the 16x16 tile Y = op(M) P: rows are
// state rows, columns the tile's state columns.
#include <hip/hip_runtime.h>

#include "qla_internal.h"

namespace qla {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));

constexpr int kTileV = 16;     // kv-view columns per workgroup
constexpr int kLdsPad = 8;     // LDS state row stride K + 8 floats: conflict-free 16-byte operand reads
constexpr int kProducers = 4;  // producer waves of the K <= 128 kernels
// K <= 128 kernels: H is loaded kHAhead steps ahead, and M_j's lines are
// warmed into L2 kMTouch steps ahead of its copy.
constexpr int kHAhead = 3;
constexpr int kMTouch = 2;
constexpr int kMoAhead = 2;    // general kernel: staged M operand reads run this many blocks ahead

// Compute sizes.  K <= 128 (every multiple of 16) runs the producer kernels
// with K/16 MFMA waves of 16 rows each.  K = 256 runs the general kernel,
// 8 MFMA waves forward and 4 backward: its backward M share is a column
// block, and 32 columns per wave make each load a whole 128-byte line per row
// (16 columns would halve that).  128 < K < 256 runs the same general kernel
// at compute size 256 with the missing rows and columns read as zeros (a
// zero-padded M and state give exactly the unpadded result in the first K
// rows).  A grouped call at K > 128 runs its forward and its backward
// groups as one launch each, with these same wave counts.
constexpr int general_waves(bool fwd) { return fwd ? 8 : 4; }
// Prefetch distance of the general kernel, in units (64-k panels) of M.
constexpr int kPrefetchUnits = 1;
constexpr int pow2_divisor(int x) { return x % 2 ? 1 : 2 * pow2_divisor(x / 2); }
// XOR swizzle of a row's 16-byte chunks in an M stage: by the row's low bits,
// as many as keep the chunk index inside the row (a power of two dividing the
// row's K/4 chunks), at most the low four.
constexpr int stage_swizzle(int kp) { return pow2_divisor(kp / 4) < 16 ? pow2_divisor(kp / 4) : 16; }

template <int K, int WAVES_, bool FWD_>
struct Shape {
    static constexpr int WAVES = WAVES_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int ROWS = K / WAVES;        // output rows per wave
    static constexpr int T = ROWS / 16;           // 16-row MFMA tiles per wave
    static constexpr int KP = K >= 256 ? 64 : K;  // k-width of one M panel
    static constexpr int NP = K / KP;             // panels per step
    static constexpr int BP = KP / 16;            // 16-wide k blocks per panel
    static constexpr int LS = K + kLdsPad;        // LDS row stride (floats)
    static constexpr int SWZ = stage_swizzle(KP); // chunk swizzle of a staged M row
    static constexpr int STATE_FLOATS = 2 * kTileV * LS;  // two state slots
    static constexpr int STAGE_FLOATS = ROWS * KP;          // one wave's M panel share
    // Forward staging slots per wave: two (the next panel is written while
    // this one is read) when they fit in the 160 KiB of LDS, else one.
    static constexpr int SS =
        (STATE_FLOATS + WAVES * 2 * STAGE_FLOATS) * 4 <= 160 * 1024 && kPrefetchUnits >= 2 ? 2 : 1;
    static constexpr int RPI = KP >= 64 ? 256 / KP : 1;    // M rows per coalesced load instruction (general kernel)
    // Prefetch distance in panels (see Tile::prefetch).
    static constexpr int D = kPrefetchUnits;
    static_assert(K % 16 == 0 && ROWS % 16 == 0, "whole 16-row tiles per wave");
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
// out is written with plain (cached) stores: with inputs streamed from HBM they
// beat non-temporal and write-through ones (a kv tile writes 64-byte halves of
// lines that L2 merges with the neighbouring tile's halves).
__device__ __forceinline__ void bstore1(__amdgpu_buffer_rsrc_t r, unsigned off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, unsigned off, f4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void st4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }

// Optional forced-delay schedule (built only into the race-test library): one
// wave per step sleeps before reading the shared state slot, another before
// writing the next one, and one producer before its copy.  Results must not
// change.
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

// PAD: the caller's head dimension kp (a multiple of 16, below K) is smaller
// than the compute size K; rows and columns kp .. K-1 of M and of the state
// are read as zeros and never written.
template <int K, int LAYOUT, int DIR, int WAVES, bool PAD = false>
struct Tile {
    using S = Shape<K, WAVES, DIR == QLA_DIR_FWD>;
    static constexpr int T = S::T, KP = S::KP, NP = S::NP, BP = S::BP, LS = S::LS;
    static constexpr bool KV = LAYOUT == QLA_LAYOUT_KV;
    static constexpr bool FWD = DIR == QLA_DIR_FWD;
    static constexpr bool STAGE = FWD;  // forward M goes through LDS staging
    // LDS: two state slots, plus one M staging slot per wave when forward.
    static constexpr int SS = S::SS;
    static constexpr int SF = S::STAGE_FLOATS;
    static constexpr int LDS_FLOATS = S::STATE_FLOATS + (STAGE ? S::WAVES * SS * SF : 0);

    // Per-lane constants of one workgroup.
    struct Lane {
        int wave, g, c, a0;
        unsigned hoff[T];  // vk: byte offsets of the lane's 16-byte H/out vectors
        unsigned hk[T][4]; // kv: byte offset of fragment element (t, r)  (kOutOfRange if masked)
        unsigned moff;     // byte offset of the lane's first M operand (backward)
        unsigned mown;     // same, for the own-row blocks in their register order (backward)
        unsigned mcoal;    // byte offset of the lane's first coalesced M chunk (forward)
        int prot, brot;    // k-order rotation of this wave: panels, then 16-k blocks in a panel
        unsigned state_bytes;
        int kp;            // the caller's K (physical row length of M and of the state)
        int mrow, mcol;    // PAD, forward: M row and column of the lane's first coalesced chunk
    };

    // Physical K, and the byte size of one M.
    static __device__ __forceinline__ int kph(const Lane& L) { return PAD ? L.kp : K; }
    static __device__ __forceinline__ unsigned mat_bytes(const Lane& L) { return (unsigned)kph(L) * kph(L) * 4u; }
    static __device__ __forceinline__ unsigned wrapb(int x) { return (unsigned)x % (unsigned)BP; }
    static __device__ __forceinline__ unsigned wrapp(int x) { return (unsigned)x % (unsigned)NP; }

    // Row of the kv view held by fragment row i of tile t: tiles are
    // contiguous 16-row blocks forward; backward they interleave with stride
    // T so that a lane's T values of one M row are adjacent in memory.
    static __device__ __forceinline__ int arow(int a0, int t, int i)
    {
        return FWD ? a0 + 16 * t + i : a0 + T * i + t;
    }

    // The accumulator computes Y (rows = state rows a) in every variant:
    // fragment element (t, r) of lane (g, c) is row a = arow(t, 4g + r),
    // column v = v0 + c.  That is also the layout the next step's MFMA
    // operand needs for those rows, so a wave's own rows go from one step to
    // the next in registers.
    // vk memory is [v][a]: a lane's 4 (forward) or 4T (backward) rows are
    // contiguous, read as 16-byte vectors; vector/component of element (t, r):
    // forward vector t, component r; backward flat index T*r + t.  kv memory
    // is [a][v]: one float per element, 16 lanes covering 64 contiguous bytes.
    static constexpr int vec_of(int t, int r) { return (KV || FWD) ? t : (T * r + t) >> 2; }
    static constexpr int comp_of(int t, int r) { return (KV || FWD) ? r : (T * r + t) & 3; }

    // wave: the wave's index among the MFMA waves that share this tile
    // (default: its index in the workgroup).
    static __device__ __forceinline__ Lane make_lane(int v0, int V, int kp = K, int wave = -1)
    {
        Lane L;
        const int lane = threadIdx.x & 63;
        L.wave = wave >= 0 ? wave : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        L.g = lane >> 4;
        L.c = lane & 15;
        L.a0 = L.wave * S::ROWS;
        L.kp = kp;
        const int kk = kph(L);
        L.state_bytes = (unsigned)kk * V * 4u;
        const bool valid = v0 + L.c < V;
#pragma unroll
        for (int i = 0; i < T; ++i) {
            const int a = FWD ? L.a0 + 16 * i + 4 * L.g : L.a0 + 4 * T * L.g + 4 * i;  // first of 4 rows
            L.hoff[i] = valid && (!PAD || a < kk) ? 4u * (unsigned)((v0 + L.c) * kk + a) : kOutOfRange;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ar = arow(L.a0, i, 4 * L.g + r);
                L.hk[i][r] = valid && (!PAD || ar < kk) ? 4u * (unsigned)(ar * V + v0 + L.c) : kOutOfRange;
            }
        }
        // Forward: M[a0 + c][4g]; backward: M[4g][a0 + T*c] (panel/block/tile offsets added per load).
        L.moff = 4u * (unsigned)(4 * L.g * kk + L.a0 + T * L.c);
        // Backward own-row block t, instruction q: k = a0 + T*(4g + q) + t.
        L.mown = 4u * (unsigned)((L.a0 + 4 * T * L.g) * kk + L.a0 + T * L.c);
        // Each wave walks the k range starting at its own rows (k = a0 ...):
        // the state of those rows is its own output, readable before the
        // other waves have written theirs.
        L.prot = (L.wave * S::ROWS / KP) % NP;
        L.brot = (L.wave * S::ROWS / 16) % BP;
        L.mrow = L.a0 + lane / (KP / 4);
        L.mcol = 4 * (lane % (KP / 4));
        L.mcoal = 4u * (unsigned)(L.mrow * kk + L.mcol);
        return L;
    }

    // Loads of one state matrix's share: T vectors (vk) or 4T floats (kv).
    static constexpr int kStateLoads = KV ? 4 * T : T;

    template <int I>
    static __device__ __forceinline__ void load_state_one(f4 (&h)[T], __amdgpu_buffer_rsrc_t r, const Lane& L)
    {
        if constexpr (KV) h[I / 4][I % 4] = bload1(r, L.hk[I / 4][I % 4]);
        else h[I] = bload4(r, L.hoff[I]);
    }

    static __device__ __forceinline__ void load_state(f4 (&h)[T], __amdgpu_buffer_rsrc_t r, const Lane& L)
    {
        if constexpr (KV) {
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) h[t][q] = bload1(r, L.hk[t][q]);
        } else {
#pragma unroll
            for (int i = 0; i < T; ++i) h[i] = bload4(r, L.hoff[i]);
        }
    }

    static __device__ __forceinline__ void store_state(__amdgpu_buffer_rsrc_t r, const f4 (&x)[T], const Lane& L)
    {
        if constexpr (KV) {
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) bstore1(r, L.hk[t][q], x[t][q]);
        } else {
            f4 ov[T];
            vecs_from_frag(ov, x);
#pragma unroll
            for (int i = 0; i < T; ++i) bstore4(r, L.hoff[i], ov[i]);
        }
    }

    // Forward M staging.  Each wave owns a private LDS slot of ROWS x KP
    // floats, laid out [row][16-byte chunk] with the chunk index XORed by
    // (row & 15) so that both the line-wise writes and the MFMA-layout reads
    // (16 rows, same chunk) spread over all banks.  The slot is private to
    // the wave and LDS executes one wave's accesses in order, so the next
    // panel's writes cannot overtake this panel's reads: no barrier needed.
    static __device__ __forceinline__ int stage_off(int row, int chunk) { return row * KP + 4 * (chunk ^ (row & (S::SWZ - 1))); }

    // MFMA operand (a, k) = M[a0 + 16t + c][p*KP + 16b + 4g + q] for one (t, b).
    static __device__ __forceinline__ f4 stage_read(const float* stage, int t, int b, const Lane& L)
    {
        return *reinterpret_cast<const f4*>(stage + stage_off(16 * t + L.c, 4 * wrapb(b + L.brot) + L.g));
    }

    // Position of k block (panel p, block b of the wave's walk) in the k range.
    static __device__ __forceinline__ int panel_of(int p, const Lane& L) { return wrapp(p + L.prot); }
    static __device__ __forceinline__ int kblock(int p, int b, const Lane& L) { return panel_of(p, L) * BP + wrapb(b + L.brot); }

    // Write the lane's fragment of the state into one LDS slot ([v][k] order):
    // element (t, r) is column v = c, row a = arow(t, 4g + r).
    static __device__ __forceinline__ void put_state(float* buf, const f4 (&x)[T], const Lane& L)
    {
        const int g = L.g, c = L.c, a0 = L.a0;
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
    static_assert(!(STAGE && SS == 2) || D >= 2, "two-slot staging stages a unit loaded two units ahead");

    // Blocks of a step, in the wave's k order: the first T blocks of panel 0
    // are the wave's own rows.  Their state operand is the wave's own output
    // of the previous step, still in registers: own block t is accumulator
    // tile t, so its k order follows the accumulator layout (forward the
    // natural one; backward k = a0 + T*(4g + q) + t, and the M operand of
    // those blocks is loaded in the same order).  Those MFMAs run while the
    // other waves' rows are still being read from LDS.
    static constexpr int kOwn = T;  // 16-k blocks of own rows
    static_assert(kOwn <= BP, "own rows fit in the first panel");
    // Forward, one panel per step, two staging slots: the first two staged
    // M operand blocks of a step are read at the end of the previous step.
    static constexpr bool kMoCarried = STAGE && SS == 2 && NP == 1;
    static constexpr int MA = kMoAhead < BP ? kMoAhead : BP;  // staged reads run MA blocks ahead

    // ---- one load / staging-write instruction at a time -------------------
    // Loads of one M panel (this wave's share): forward, T*BP whole-line
    // instructions (instruction i covers rows i*RPI .. i*RPI + RPI - 1 of the
    // share); backward, 4*BP T-wide instructions (one per (b, q)).
    static constexpr int kPanelLoads = FWD ? T * BP : 4 * BP;

    template <int I, int TP>
    static __device__ __forceinline__ void load_m(f4 (&m)[T][BP], __amdgpu_buffer_rsrc_t Mr, const Lane& L)
    {
        const int pa = panel_of(TP, L);
        const int kk = kph(L);
        if constexpr (STAGE) {
            unsigned off = L.mcoal + 4u * (unsigned)(I * S::RPI * kk + pa * KP);
            if constexpr (PAD)
                if (L.mrow + I * S::RPI >= kk || pa * KP + L.mcol >= kk) off = kOutOfRange;
            m[I / BP][I % BP] = bload4(Mr, off);
        } else {
            // operand (a, k) = M[k][a], a = a0 + T*c + t; k = 16*kblock + 4g + q,
            // or the own-row order for the first kOwn blocks of panel 0
            constexpr int b = I / 4, q = I % 4;
            const bool own = TP == 0 && b < kOwn;
            unsigned off = own ? L.mown + 4u * (unsigned)((T * q + b) * kk)
                               : L.moff + 4u * (unsigned)((pa * KP + 16 * (int)wrapb(b + L.brot) + q) * kk);
            if constexpr (PAD) {
                const int k = own ? L.a0 + T * (4 * L.g + q) + b : pa * KP + 16 * (int)wrapb(b + L.brot) + 4 * L.g + q;
                if (k >= kk || L.a0 + T * L.c >= kk) off = kOutOfRange;
            }
            if constexpr (T == 1) {
                m[0][b][q] = bload1(Mr, off);
            } else if constexpr (T == 2) {
                const f2 x = bload2(Mr, off);
                m[0][b][q] = x[0];
                m[1][b][q] = x[1];
            } else {
                const f4 x = bload4(Mr, off);
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
    };

    // Issue prefetch loads [LO, HI) of the target unit: M instructions first,
    // then (on a step's first panel) the T vectors of H.
    template <int LO, int HI, int TLS, int TP>
    static __device__ __forceinline__ void issue_loads(const Prefetch& pf, f4 (&m)[R][T][BP], f4 (&h)[RH][T],
                                                       const Lane& L)
    {
        if constexpr (LO < HI) {
            if constexpr (LO < kPanelLoads)
                load_m<LO, TP>(m[(TLS * NP + TP) % R], pf.Mr, L);
            else
                load_state_one<LO - kPanelLoads>(h[TLS % RH], pf.Hr, L);
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

    static constexpr int kLinesT = K * K * 4 / 128;  // 128-byte lines of one M
    static constexpr int kTouchT = (kLinesT + 64 * S::WAVES - 1) / (64 * S::WAVES);
    // Steps ahead of the touch: at K = 256 one step before the prefetch (two
    // steps' worth of M, H and out for two chains already fill much of an
    // XCD's 4 MiB L2; warming earlier lets lines fall out before all 16 tiles
    // have loaded them), elsewhere two.
    static constexpr int TD = (D + NP - 1) / NP + (K >= 256 ? 1 : 2);

    // Working registers, carried from step to step.
    struct StepCtx {
        f4 acc[T];
        f4 own[T];     // the wave's own rows of the current state (operand of the own blocks)
        f4 pv[K / 16]; // state operand blocks read from LDS
        f4 mo[MA + 1][T];  // forward: staged M operand, read MA blocks ahead
        f4 mh[MA][T];      // forward: the next panel's first MA blocks of it
        const float* cur;
        const float* st_cur;
        float* st_next;
        __amdgpu_buffer_rsrc_t out_prev;  // out_j of the previous step (empty at step 0)
        float touched[F][kTouchT];        // cache warm-up loads, consumed F steps later
        int tile, tiles;
    };

    // L2 warm-up of M ahead of the register prefetch (which runs D units, so
    // D / NP steps, ahead): in step s the waves of the chain's workgroups touch
    // each 128-byte line of M for step s + TD once (one 4-byte load per line:
    // wave w of tile t takes lines t + tiles*(w + WAVES*(lane + 64k))).  The
    // value is consumed F steps later, when the compiler's wait for it is long
    // satisfied; lanes past the end use an out-of-range offset.
    static __device__ __forceinline__ void touch_ahead(float (&y)[kTouchT], const Chain& C, int s, const StepCtx& X,
                                                       const Lane& L)
    {
        const bool live = s < C.n_seg;
        const int kk = kph(L);
        const int lines = PAD ? kk * kk * 4 / 128 : kLinesT;
        const __amdgpu_buffer_rsrc_t r = rsrc(C.M + (size_t)seg(C, live ? s : 0) * kk * kk, live ? mat_bytes(L) : 0u);
#pragma unroll
        for (int k = 0; k < kTouchT; ++k) {
            const int line = X.tile + X.tiles * (L.wave + S::WAVES * ((int)(threadIdx.x & 63) + 64 * k));
            y[k] = bload1(r, line < lines ? 128u * (unsigned)line : kOutOfRange);
        }
    }

    // The staged M operand of a panel's first MA blocks.
    static __device__ __forceinline__ void read_mo_head(f4 (&mh)[MA][T], const float* st, const Lane& L)
    {
#pragma unroll
        for (int b = 0; b < MA; ++b)
#pragma unroll
            for (int t = 0; t < T; ++t) mh[b][t] = stage_read(st, t, b, L);
    }

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
        constexpr int NL = kPanelLoads + (TP == 0 ? kStateLoads : 0);
        constexpr int l0 = NL * B / BP, l1 = NL * (B + 1) / BP;
        // Staging writes of the next unit go out over the first WB blocks, so
        // that the LDS queue has drained them well before the step's end.
        constexpr int NW = (STAGE && SS == 2) ? T * BP : 0;
        constexpr int WB = BP > 2 ? BP - 2 : BP;
        constexpr int w0 = B < WB ? NW * B / WB : NW, w1 = B < WB ? NW * (B + 1) / WB : NW;
        constexpr int nr = (STAGE && B + MA < BP) ? T : 0;
        // After the last staging write: the next step's first staged operand
        // blocks, early enough to stay off the step's closing LDS wait.
        constexpr int nmo = (kMoCarried && P == NP - 1 && B == (WB < BP ? WB : BP - 1)) ? MA * T : 0;

        auto mfma = [&](int q) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                float pk;
                if constexpr (P == 0 && B < kOwn) pk = X.own[B][q];
                else pk = X.pv[P * BP + B][q];
                const float mk = STAGE ? X.mo[B % (MA + 1)][t][q] : m[slot][t][B][q];
                X.acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(mk, pk, X.acc[t], 0, 0, 0);
            }
        };
        mfma(0);
        mfma(1);
        if constexpr (nr > 0) {
#pragma unroll
            for (int t = 0; t < T; ++t) X.mo[(B + MA) % (MA + 1)][t] = stage_read(X.st_cur, t, B + MA, L);
        }
        issue_loads<l0, l1, TLS, TP>(pf, m, h, L);
        if constexpr (NW > 0) issue_writes<w0, w1>(X.st_next, m[(LSX * NP + P + 1) % R]);
        mfma(2);
        mfma(3);
        if constexpr (nmo > 0) read_mo_head(X.mh, X.st_next, L);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * T, 0);                                // MFMA
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);             // DS read
        if constexpr (l1 > l0) __builtin_amdgcn_sched_group_barrier(0x020, l1 - l0, 0);       // VMEM read
        if constexpr (w1 > w0) __builtin_amdgcn_sched_group_barrier(0x200, w1 - w0, 0);       // DS write
        if constexpr (nmo > 0) __builtin_amdgcn_sched_group_barrier(0x100, nmo, 0);           // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * T, 0);                                // MFMA
        __builtin_amdgcn_sched_barrier(0);
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
        const Prefetch pf{rsrc(C.M + (size_t)tj * kph(L) * kph(L), live ? mat_bytes(L) : 0u),
                          rsrc(C.H + (size_t)tj * (L.state_bytes / 4), live ? L.state_bytes : 0u)};
        // Forward: this panel's M is read from staging slot (unit & 1),
        // written during the previous panel (two slots) or just below (one).
        // The next panel goes into the other slot, which the previous panel
        // last read: this wave issued those reads before these writes, and LDS
        // runs one wave's accesses in order.
        const int unit = s * NP + P;
        X.st_cur = stage + (SS == 2 ? (unit & 1) * SF : 0);
        X.st_next = stage + (SS == 2 ? ((unit + 1) & 1) * SF : 0);

        // State operand from LDS: all blocks but panel 0's own rows.
        read_pv<P, (P == 0 ? kOwn : 0), BP>(X.pv, X.cur, L);
        // The previous step's out_j leaves after the barrier, off the path
        // that leads to it.
        if constexpr (P == 0) store_state(X.out_prev, X.own, L);
        if constexpr (STAGE && SS == 1) issue_writes<0, T * BP>(stage, m[slot]);
        if constexpr (STAGE && !(P == 0 && kMoCarried)) read_mo_head(X.mh, X.st_cur, L);
        if constexpr (STAGE) {
#pragma unroll
            for (int b = 0; b < MA; ++b)
#pragma unroll
                for (int t = 0; t < T; ++t) X.mo[b][t] = X.mh[b][t];
        }
        __builtin_amdgcn_sched_barrier(0);
        block<LSX, P, 0>(X, pf, m, h, L);
        if constexpr (P + 1 < NP) panel<LSX, P + 1>(s, X, C, m, h, stage, L);
    }

    // One segment step with compile-time local index LSX (position in the
    // unrolled block).  The step opens with the barrier that publishes the
    // state rows every wave wrote to LDS slot s & 1 at the end of step s-1
    // (each wave first waits for its own LDS traffic), then reads the other
    // waves' rows from that slot; its own rows it already holds, and it
    // stores them as out of step s-1.  It ends by writing its rows of the new
    // state to slot (s + 1) & 1.  That slot was last read during step s-1,
    // and every wave finished those reads (the wait before the barrier)
    // before any wave passed the barrier that opens step s.
    template <int LSX>
    static __device__ __forceinline__ void step(int s, StepCtx& X, const Chain& C, f4 (&m)[R][T][BP],
                                                f4 (&h)[RH][T], float* lds, const Lane& L)
    {
        s = __builtin_amdgcn_readfirstlane(s);  // uniform: keeps the step's descriptors scalar
        float* nxt = lds + ((s + 1) & 1) * (kTileV * LS);
        float* stage = lds + S::STATE_FLOATS + L.wave * SS * SF;
        const int jp = s > 0 ? seg(C, s - 1) : 0;
        X.out_prev = rsrc(C.out + (size_t)jp * (L.state_bytes / 4), s > 0 ? L.state_bytes : 0u);

        __builtin_amdgcn_sched_barrier(0);
        lds_handoff();
        debug_delay(L.wave, s, 0);
        X.cur = lds + (s & 1) * (kTileV * LS);
#pragma unroll
        for (int t = 0; t < T; ++t) X.acc[t] = f4{0.f, 0.f, 0.f, 0.f};
        panel<LSX, 0>(s, X, C, m, h, stage, L);

        // Correct: P = Y + X(H_j); hand the state to the next step (LDS for
        // the other waves, registers for this one, which also emits it).
        f4 hx[T];
        frag_from_vecs(hx, h[LSX % RH]);
#pragma unroll
        for (int t = 0; t < T; ++t) X.acc[t] += hx[t];
        debug_delay(L.wave, s, 1);
        put_state(nxt, X.acc, L);
#pragma unroll
        for (int t = 0; t < T; ++t) X.own[t] = X.acc[t];
#pragma unroll
        for (int k = 0; k < kTouchT; ++k) asm volatile("" ::"v"(X.touched[LSX][k]));
        touch_ahead(X.touched[LSX], C, s + TD, X, L);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Remaining steps after the unrolled loop (fewer than F), straight-line.
    template <int LSX>
    static __device__ __forceinline__ void tail(int s, int rem, StepCtx& X, const Chain& C, f4 (&m)[R][T][BP],
                                                f4 (&h)[RH][T], float* lds, const Lane& L)
    {
        if constexpr (LSX < F - 1) {
            if (rem > LSX) {
                step<LSX>(s + LSX, X, C, m, h, lds, L);
                tail<LSX + 1>(s, rem, X, C, m, h, lds, L);
            }
        }
    }

    // Prologue loads: units LO .. HI-1 (and the H of the steps they start).
    template <int LO, int HI>
    static __device__ __forceinline__ void prologue(const Chain& C, f4 (&m)[R][T][BP], f4 (&h)[RH][T],
                                                    const Lane& L)
    {
        if constexpr (LO < HI) {
            constexpr int TLS = LO / NP, TP = LO % NP;
            const bool live = TLS < C.n_seg;
            const int tj = live ? seg(C, TLS) : 0;
            const Prefetch pf{rsrc(C.M + (size_t)tj * kph(L) * kph(L), live ? mat_bytes(L) : 0u),
                              rsrc(C.H + (size_t)tj * (L.state_bytes / 4), live ? L.state_bytes : 0u)};
            issue_loads<0, kPanelLoads + (TP == 0 ? kStateLoads : 0), TLS, TP>(pf, m, h, L);
            prologue<LO + 1, HI>(C, m, h, L);
        }
    }

    // Chain `chain` of a call whose chains all have n_seg segments.
    static __device__ __forceinline__ void run(const float* H, const float* M, const float* S0, float* out,
                                               int n_seg, int V, size_t chain, int tile, float* lds, int kp = K)
    {
        const size_t kk = PAD ? kp : K;
        const size_t state = kk * V;
        const Chain C{M + chain * (size_t)n_seg * kk * kk, H + chain * state * n_seg, out + chain * state * n_seg,
                      n_seg};
        run_chain(C, S0 ? S0 + chain * state : nullptr, V, tile, lds, kp);
    }

    // One chain given by its base pointers and segment count; S0c is its
    // initial state or NULL.  A chain without segments runs no step: every
    // global access below is then out of its buffer resource's range and
    // does nothing (kept branch-free: an early return here costs the compiler
    // its knowledge that the descriptors are uniform).
    static __device__ __forceinline__ void run_chain(const Chain& C, const float* S0c, int V, int tile, float* lds,
                                                     int kp = K)
    {
        const Lane L = make_lane(tile * kTileV, V, kp);

        f4 m[R][T][BP];
        f4 h[RH][T];
        StepCtx X;
        X.tile = tile;
        X.tiles = (V + kTileV - 1) / kTileV;
#pragma unroll
        for (int i = 0; i < F; ++i)
#pragma unroll
            for (int k = 0; k < kTouchT; ++k) X.touched[i][k] = 0.f;
        // Prologue.  A CU's vector memory path takes about 64 bytes per clock,
        // and a wave stalls at a load it cannot queue, so the loads go out in
        // the order they are needed: the initial state and the first unit of
        // M (with H of step 0); that unit's staging and the initial state's
        // hand-off; only then the rest of the prefetch distance, which the
        // first steps' work covers.
        f4 sv[T];
        load_state(sv, rsrc(S0c ? S0c : C.H, S0c ? L.state_bytes : 0u), L);
        prologue<0, 1>(C, m, h, L);
        frag_from_vecs(X.own, sv);
        put_state(lds, X.own, L);
        float* stage0 = lds + S::STATE_FLOATS + L.wave * SS * SF;
        if constexpr (STAGE && SS == 2) issue_writes<0, T * BP>(stage0, m[0]);
        if constexpr (kMoCarried) read_mo_head(X.mh, stage0, L);
        prologue<1, D>(C, m, h, L);

        int s = 0;
        for (; s + F <= C.n_seg; s += F) {
            step<0>(s, X, C, m, h, lds, L);
            if constexpr (F > 1) step<1 % F>(s + 1, X, C, m, h, lds, L);
            if constexpr (F > 2) step<2 % F>(s + 2, X, C, m, h, lds, L);
            if constexpr (F > 3) step<3 % F>(s + 3, X, C, m, h, lds, L);
            if constexpr (F > 4) step<4 % F>(s + 4, X, C, m, h, lds, L);
            if constexpr (F > 5) step<5 % F>(s + 5, X, C, m, h, lds, L);
        }
        tail<0>(s, C.n_seg - s, X, C, m, h, lds, L);
        const bool any = C.n_seg > 0;
        store_state(rsrc(C.out + (size_t)seg(C, any ? C.n_seg - 1 : 0) * (L.state_bytes / 4), any ? L.state_bytes : 0u),
                    X.own, L);
    }
};

// K <= 128 (any multiple of 16), both directions: producer waves and K/16
// MFMA waves of 16 rows each.  Waves CW .. CW+PW-1 of
// the workgroup only move M: together they copy each M_j whole from global
// memory into one of two LDS stages with 16-byte LDS-DMA buffer loads (the
// data never passes through registers; each producer issues an equal share
// of the copies, so that enough of them are in flight to cover the memory
// latency), issue the L2 warm-up loads for later steps, wait for the copies,
// and join the step barrier.
// Waves 0 .. CW-1 compute as above, reading their operand of M from the
// stage: forward their rows of M (one 16-byte read per 16-k block), backward
// the same columns of M, which are the rows of M^T (four 4-byte reads per
// block; the copy cannot transpose).  They issue no M loads, so their
// instruction streams are MFMAs and LDS reads.  One barrier per step orders everything: after the barrier that
// opens step s the producer refills the stage of unit s-1 with unit s+1
// (every MFMA wave finished reading it before arriving), and unit s+1 has
// landed before the producer arrives at the barrier that opens step s+1.
// The stage holds M row-major with each row's 16-byte chunks XOR-swizzled
// by the row's low bits (four of them when the row has at least 16 chunks,
// K >= 64), so at K = 64 and 128 the whole-row copy and the MFMA-layout reads
// of either direction are free of bank conflicts (backward, the four rows a
// read instruction touches differ in bits 2-3 of k, which moves their chunks
// to distinct banks).
template <int K, int LAYOUT, int DIR = QLA_DIR_FWD, int G = 1>
struct DmaChain {
    static_assert(K % 16 == 0 && K >= 16 && K <= 128, "producer kernels cover K = 16 .. 128");
    static_assert(G == 1 || (G == 2 && K % 32 == 0), "two groups of waves with 32 rows each");
    static constexpr int CW = K / 16;                  // MFMA waves
    static constexpr int CWG = CW / G;                 // MFMA waves per group, 16 G rows each
    static constexpr int PW = kProducers;              // producer waves
    using Tl = Tile<K, LAYOUT, QLA_DIR_FWD, CWG>;
    using S = typename Tl::S;
    using Lane = typename Tl::Lane;
    using Chain = typename Tl::Chain;
    // Segment of step s: forward in order, backward in reverse.
    static __device__ __forceinline__ int sg(const Chain& C, int s) { return DIR == QLA_DIR_FWD ? s : C.n_seg - 1 - s; }
    // Staged operand of (t, block b): forward M[a0 + 16t + c][k] (the wave's
    // rows, one 16-byte read); backward M[k][a0 + 16t + c] (a column, four
    // 4-byte reads), k = 16 kb + 4g + q.
    template <int NT>
    static __device__ __forceinline__ f4 rd(const float* st, int t, int b, const Lane& L, const int (&X_tofs)[NT][4])
    {
        if constexpr (DIR == QLA_DIR_FWD) {
            return Tl::stage_read(st, t, b, L);
        } else {
            // k & 15 = 4g + q does not depend on the block, so the lane's four
            // byte offsets per row tile (tofs) are fixed; the block adds a
            // uniform 16 K-float step.
            const int kofs = __builtin_amdgcn_readfirstlane((int)Tl::wrapb(b + L.brot) * 16 * K * 4);
            const char* sb = reinterpret_cast<const char*>(st) + kofs;
            f4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const float*>(sb + X_tofs[t][0] + q * K * 4);
            return v;
        }
    }
    static constexpr int T = S::T, BP = S::BP, LS = S::LS;
    static_assert(S::NP == 1, "one panel per step");
    static constexpr int kOwn = T;
    static constexpr int MA = 2;                      // staged reads run two blocks ahead
    static constexpr int STAGE = K * K;               // floats per M stage
    static constexpr int WARM = S::STATE_FLOATS + 2 * STAGE;  // the sink the warm-up loads land in
    static constexpr int kDmaAll = K * K / 256;              // 1 KiB copies per M
    // The sink: 64 floats for the 4-byte warm-ups, 256 when the producers'
    // copy counts differ and the spare copies (1 KiB, of nothing) land there.
    static constexpr int LDS_FLOATS = WARM + (kDmaAll % kProducers ? 256 : 64);
    static constexpr int SWZ = S::SWZ;                // chunk swizzle of a stage row
    // The XOR applied to a stage row's chunk index.  Forward: the row's low
    // bits (16 rows of one 16-byte read each spread over all banks).
    // Backward: the row's bits 2 and up, the low two cleared, so the four
    // rows 4g .. 4g+3 that one lane reads per 16-k block share it: their
    // words lie exactly one row apart and the compiler pairs them into
    // two-address LDS reads (half the read instructions).  A 64-lane read then
    // hits every bank twice, the minimum for 256 bytes.
    static __device__ __forceinline__ int swz_row(int row)
    {
        return DIR == QLA_DIR_FWD ? (row & (SWZ - 1)) : ((row & ~3) & (SWZ - 1));
    }
    static constexpr int kDma = kDmaAll;
    static constexpr int kPer = (kDma + PW - 1) / PW; // copies per producer (the last ones may be empty)
    static constexpr int HA = kHAhead;                // H is loaded HA steps ahead
    static constexpr int HR = HA + 1;                 // H register slots
    static constexpr unsigned kMatBytes = (unsigned)K * K * 4u;

    struct Ctx {
        f4 acc[T];
        f4 own[T];
        f4 pv[K / 16];
        f4 mo[MA + 1][T];
        const float* cur;
        const float* st;
        __amdgpu_buffer_rsrc_t out_prev;
        int tofs[T][4];  // backward: byte offsets of the lane's staged column reads, per row tile
    };

    // L2 warm-up loads, issued by the producers right after each step's copy.
    // A CU returns vector-memory data in issue order, so a load that misses
    // to HBM holds up every load issued after it on that CU, the next copy of
    // M included.  The data of step s+1 is therefore brought into L2 ahead of
    // time by one 4-byte load per 128-byte line, each issued right behind a
    // copy so that it has a whole step to return before the next copy goes
    // out: the M_j lines (the chain's workgroups sit on one XCD and copy the
    // same M_j, so together they load each line once: producer p of tile t
    // takes lines t + tiles*(p + PW*lane)), and the lines of this tile's H_j
    // one step before the MFMA waves load it.  The loaded words land in a
    // 256-byte LDS area nothing reads; lanes past the end use an out-of-range
    // offset and load nothing.
    using lds_ptr = __attribute__((address_space(3))) void*;
    static constexpr int kLines = K * K * 4 / 128;
    static __device__ __forceinline__ void warm_m(const Chain& C, float* sink, int s, int p, int tile, int tiles)
    {
        const bool live = s < C.n_seg;
        const __amdgpu_buffer_rsrc_t r = rsrc(C.M + (size_t)sg(C, live ? s : 0) * K * K, live ? kMatBytes : 0u);
        const int line = tile + tiles * (p + PW * (int)(threadIdx.x & 63));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)sink, 4, line < kLines ? 128 * line : (int)kOutOfRange,
                                                 0, 0, 0);
    }
    // kv: one word in each row's 64-byte piece of the tile (rows p + PW*lane).
    // The piece shares its 128-byte line with the neighbouring tile's, which
    // sits on the same XCD, so of a pair of tiles each warms every other row
    // (a tile without a neighbour warms all).  vk: the tile's rows are one
    // contiguous block of 16 K floats (64 K bytes, a multiple of 128): one
    // word in each of its K/2 lines.
    static __device__ __forceinline__ void warm_h(const Chain& C, float* sink, int s, int p, int tile, int V)
    {
        const bool live = s < C.n_seg;
        const unsigned bytes = (unsigned)K * V * 4u;
        const __amdgpu_buffer_rsrc_t r = rsrc(C.H + (size_t)sg(C, live ? s : 0) * (bytes / 4), live ? bytes : 0u);
        const int idx = p + PW * (int)(threadIdx.x & 63);
        unsigned off = kOutOfRange;
        if constexpr (LAYOUT == QLA_LAYOUT_KV) {
            const int tiles = (V + kTileV - 1) / kTileV;
            const bool mine = (tile ^ 1) >= tiles || ((idx ^ tile) & 1) == 0;
            if (idx < K && mine) off = 4u * (unsigned)(idx * V) + 64u * (unsigned)tile;
        } else {
            if (idx < K / 2) off = 64u * (unsigned)K * (unsigned)tile + 128u * (unsigned)idx;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)sink, 4, (int)off, 0, 0, 0);
    }

    // ---- producer ---------------------------------------------------------
    // Copy M_j into a stage: copy i fills stage floats [256 i, 256 i + 256);
    // lane l's 16 bytes land at float 256 i + 4 l = (row, swizzled chunk).
    // Producer p issues copies p, p + PW, p + 2 PW, ... (K*K/256 of them in
    // all).  When PW does not divide that, a producer past the end issues a
    // copy of nothing (an out-of-range source) into the sink, so every
    // producer runs the same straight-line instruction sequence.
    static __device__ __forceinline__ void dma_unit(const float* Mj, float* stage, float* sink, int p)
    {
        const __amdgpu_buffer_rsrc_t r = rsrc(Mj, kMatBytes);
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = k * PW + p;
            const bool real = kDma % PW == 0 || i < kDma;
            const int q = 256 * i + 4 * lane;
            const int row = q / K, chunk = (q % K) / 4;
            const int src = row * K + 4 * (chunk ^ swz_row(row));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(real ? stage + 256 * i : sink),
                                                     16, real ? 4 * src : (int)kOutOfRange, 0, 0, 0);
        }
    }

    // Each step: the copy, then the warm-ups for M_{s+1+kMTouch} and for
    // the H the MFMA waves load next step; the barrier waits for the copy
    // only (vmcnt counts in issue order, so leaving the warm-ups outstanding
    // still covers every copy instruction).
    // The wait is correct only if the warm-ups are issued after every copy:
    // a compiler barrier keeps both the IR passes and the machine scheduler
    // from moving them across (tests/test_kernel_isa.py checks the built code).
    static __device__ __forceinline__ void copies_before_warmups()
    {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
    static constexpr int kWarmPerStep = 2;  // warm-up instructions per producer and step
    static __device__ __forceinline__ void producer(const Chain& C, float* lds, int p, int tile, int V)
    {
        float* stages = lds + S::STATE_FLOATS;
        float* sink = lds + WARM;
        const int tiles = (V + kTileV - 1) / kTileV;
        dma_unit(C.M + (size_t)sg(C, 0) * K * K, stages, sink, p);
        copies_before_warmups();
#pragma unroll
        for (int u = 1; u <= kMTouch; ++u) warm_m(C, sink, u, p, tile, tiles);
        warm_h(C, sink, HA, p, tile, V);
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kMTouch + 1) : "memory");
        for (int s = 0; s + 1 < C.n_seg; ++s) {
            debug_delay(p, s, 2);  // a late copy: the MFMA waves must wait for it at the barrier
            dma_unit(C.M + (size_t)sg(C, s + 1) * K * K, stages + ((s + 1) & 1) * STAGE, sink, p);
            copies_before_warmups();
            warm_m(C, sink, s + 1 + kMTouch, p, tile, tiles);
            warm_h(C, sink, s + 1 + HA, p, tile, V);
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kWarmPerStep) : "memory");
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // Two groups (G = 2): workgroup tp carries tiles tp and tp + pairs of one
    // chain, one per group of MFMA waves, and a barrier falls every half
    // step.  (In the kv layout a 128-byte line of a row holds the 64-byte
    // pieces of tiles 2m and 2m + 1: they belong to the same group of two
    // neighbouring workgroups, which run in phase on one XCD, so L2 merges
    // the halves of each out line as it does for single tiles.  Tiles 2 tp and
    // 2 tp + 1 in one workgroup would write them half a step apart, and a
    // third more bytes reached memory.)  Group 0 runs step s from barrier 2s to barrier 2s+2, group 1 from
    // 2s+1 to 2s+3.  Both read M_s from stage s&1, so M_j (j >= 2) may
    // overwrite M_{j-2} only after barrier 2j-1, where group 1 finishes step
    // j-2, and must have landed by barrier 2j, where group 0 starts step j:
    // the producers copy it between those two barriers.  M_0 is copied
    // before barrier 0 and M_1 (stage 1, unused until then) between barriers
    // 0 and 1.  The warm-ups ride behind each copy as above: the lines of
    // M_{j+kPairTouch} and the two tiles' H lines of step j+HA.  A step here
    // takes about twice as long as a single tile's, and twice as many chains
    // share an XCD's L2, so M is warmed one step ahead (two measured 1.2-1.5x
    // the algorithmic reads: lines fell out of L2 before their copy).
    static constexpr int kPairTouch = 1;
    // Slot i = p + PW*lane: i < 128 tile A, 128 .. 255 tile B.  kv: one word in
    // each row's 64-byte piece of the tile, every other row when the partner
    // tile exists (its workgroup warms the rest of the 128-byte lines); vk:
    // one word in each of the tile's K/2 lines.
    static __device__ __forceinline__ void warm_h_pair(const Chain& C, float* sink, int s, int p, int tA, int tB,
                                                       int V)
    {
        const bool live = s < C.n_seg;
        const unsigned bytes = (unsigned)K * V * 4u;
        const __amdgpu_buffer_rsrc_t r = rsrc(C.H + (size_t)sg(C, live ? s : 0) * (bytes / 4), live ? bytes : 0u);
        const int i = p + PW * (int)(threadIdx.x & 63);
        const int t = i < 128 ? tA : tB;
        const int j = i & 127;
        unsigned off = kOutOfRange;
        if constexpr (LAYOUT == QLA_LAYOUT_KV) {
            const int tiles = (V + kTileV - 1) / kTileV;
            const bool partner = (t ^ 1) < tiles;
            const int row = partner ? 2 * j + (t & 1) : j;
            if (row < K && (partner ? j < K / 2 : true)) off = 4u * (unsigned)(row * V) + 64u * (unsigned)t;
        } else {
            if (j < K / 2) off = 64u * (unsigned)K * (unsigned)t + 128u * (unsigned)j;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)sink, 4, (int)off, 0, 0, 0);
    }

    static __device__ __forceinline__ void copy_unit(const Chain& C, float* lds, int j, int p, int tp, int pairs,
                                                     int V)
    {
        float* sink = lds + WARM;
        dma_unit(C.M + (size_t)sg(C, j) * K * K, lds + S::STATE_FLOATS + (j & 1) * STAGE, sink, p);
        copies_before_warmups();
        warm_m(C, sink, j + kPairTouch, p, tp, pairs);
        warm_h_pair(C, sink, j + HA, p, tp, tp + pairs, V);
    }

    static __device__ __forceinline__ void producer_pair(const Chain& C, float* lds, int p, int tp, int V)
    {
        float* sink = lds + WARM;
        const int pairs = ((V + kTileV - 1) / kTileV + 1) / 2;
        dma_unit(C.M + (size_t)sg(C, 0) * K * K, lds + S::STATE_FLOATS, sink, p);
        copies_before_warmups();
#pragma unroll
        for (int u = 1; u <= kPairTouch; ++u) warm_m(C, sink, u, p, tp, pairs);
        warm_h_pair(C, sink, HA, p, tp, tp + pairs, V);
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kPairTouch + 1) : "memory");
        // after barrier k, before barrier k + 1 (k = 0 .. 2n-1)
        for (int k = 0; k < 2 * C.n_seg; ++k) {
            const int j = k == 0 ? 1 : ((k & 1) && k >= 3 ? (k + 1) / 2 : -1);
            if (j >= 1 && j < C.n_seg) {
                debug_delay(p, j, 2);  // a late copy: both groups must wait for it at the barrier
                copy_unit(C, lds, j, p, tp, pairs, V);
                asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kWarmPerStep) : "memory");
            } else {
                asm volatile("s_barrier" ::: "memory");
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // ---- MFMA waves -------------------------------------------------------
    // The step's global accesses go out between MFMA blocks late in the
    // step: out of step s-1 before block kStoreAt, H of step s+HA (already
    // warmed into L2 by the producers) before block kLoadAt.  Right after the
    // barrier the producers fill the CU's vector memory queue, and an access
    // waiting for a slot there holds up this wave; late in the step the queue
    // has drained, and issuing them between blocks rather than all after the
    // last one lets the other wave's MFMAs cover their issue.  With fewer
    // than eight blocks (K < 128) the points fall on the nearest block
    // boundaries, with one block both before it.
    static constexpr int kStoreAt = 5 * BP / 8;
    static constexpr int kLoadAt = 7 * BP / 8 > kStoreAt ? 7 * BP / 8 : kStoreAt;
    static constexpr int kFirstReads = MA < BP ? MA : BP;  // staged operand blocks read right after the barrier

    // MFMA blocks B .. E-1 (none if B >= E).
    template <int B, int E = BP>
    static __device__ __forceinline__ void blocks(Ctx& X, const Lane& L)
    {
      if constexpr (B < E) {
        // LDS read instructions of one staged operand block: one 16-byte read
        // forward, four 4-byte reads backward (all placed after the block's
        // second MFMA, so each has six MFMAs to land)
        constexpr int nr = B + MA < BP ? T * (DIR == QLA_DIR_FWD ? 1 : 4) : 0;
        auto mfma = [&](int q) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                float pk;
                if constexpr (B < kOwn) pk = X.own[B][q];
                else pk = X.pv[B][q];
                X.acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(X.mo[B % (MA + 1)][t][q], pk, X.acc[t], 0, 0, 0);
            }
        };
        mfma(0);
        mfma(1);
        if constexpr (nr > 0) {
#pragma unroll
            for (int t = 0; t < T; ++t) X.mo[(B + MA) % (MA + 1)][t] = rd(X.st, t, B + MA, L, X.tofs);
        }
        mfma(2);
        mfma(3);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * T, 0);
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * T, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (B + 1 < E) blocks<B + 1, E>(X, L);
      }
    }

    // Step s (LSX = s % HR selects the H register slot).  Barrier; operand
    // reads (first staged M blocks, the other waves' state rows); the MFMAs
    // accumulating onto X(H_j), with out of step s-1 and H of step s+HA
    // issued between the last blocks; the new state into the next state slot
    // and the own-row registers.
    template <int LSX>
    static __device__ __forceinline__ void step(int s, Ctx& X, const Chain& C, f4 (&h)[HR][T], float* lds,
                                                const Lane& L)
    {
        s = __builtin_amdgcn_readfirstlane(s);  // uniform: keeps the step's descriptors scalar
        float* nxt = lds + ((s + 1) & 1) * (kTileV * LS);
        const int jp = s > 0 ? sg(C, s - 1) : 0;
        X.out_prev = rsrc(C.out + (size_t)jp * (L.state_bytes / 4), s > 0 ? L.state_bytes : 0u);
        const bool live = s + HA < C.n_seg;
        const __amdgpu_buffer_rsrc_t Hr =
            rsrc(C.H + (size_t)(live ? sg(C, s + HA) : 0) * (L.state_bytes / 4), live ? L.state_bytes : 0u);

        __builtin_amdgcn_sched_barrier(0);
        lds_handoff();
        debug_delay(L.wave, s, 0);
        X.cur = lds + (s & 1) * (kTileV * LS);
        X.st = lds + S::STATE_FLOATS + (s & 1) * STAGE + (DIR == QLA_DIR_FWD ? L.a0 * K : 0);
#pragma unroll
        for (int b = 0; b < kFirstReads; ++b)
#pragma unroll
            for (int t = 0; t < T; ++t) X.mo[b][t] = rd(X.st, t, b, L, X.tofs);
        Tl::template read_pv<0, kOwn, BP>(X.pv, X.cur, L);
        // The accumulator starts at X(H_j) (loaded HA steps ago), so the new
        // state is ready as soon as the last MFMA retires.
        {
            f4 hx[T];
            Tl::frag_from_vecs(hx, h[LSX]);
#pragma unroll
            for (int t = 0; t < T; ++t) X.acc[t] = hx[t];
        }
        __builtin_amdgcn_sched_barrier(0);
        blocks<0, kStoreAt>(X, L);
        Tl::store_state(X.out_prev, X.own, L);
        __builtin_amdgcn_sched_barrier(0);
        blocks<kStoreAt, kLoadAt>(X, L);
        Tl::load_state(h[(LSX + HA) % HR], Hr, L);
        __builtin_amdgcn_sched_barrier(0);
        blocks<kLoadAt, BP>(X, L);

        debug_delay(L.wave, s, 1);
        Tl::put_state(nxt, X.acc, L);
#pragma unroll
        for (int t = 0; t < T; ++t) X.own[t] = X.acc[t];
        __builtin_amdgcn_sched_barrier(0);
    }

    template <int LSX>
    static __device__ __forceinline__ void tail(int s, Ctx& X, const Chain& C, f4 (&h)[HR][T], float* lds,
                                                const Lane& L)
    {
        if constexpr (LSX < HR - 1) {
            if (s + LSX < C.n_seg) {
                step<LSX>(s + LSX, X, C, h, lds, L);
                tail<LSX + 1>(s, X, C, h, lds, L);
            }
        }
    }

    // Backward: the lane's byte offsets of its staged column reads, row tile
    // t, instruction q (row k = 4g + q of a 16-k block, column a0 + 16t + c).
    static __device__ __forceinline__ void init_tofs(Ctx& X, const Lane& L)
    {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (DIR != QLA_DIR_FWD) {
                    const int col = L.a0 + 16 * t + L.c;
                    const int r = 4 * L.g + q;
                    X.tofs[t][q] = 4 * (r * K + 4 * ((col >> 2) ^ swz_row(r)) + (col & 3));
                } else {
                    X.tofs[t][q] = 0;
                }
            }
    }

    static __device__ __forceinline__ void consumer(const Chain& C, const float* S0c, float* lds, int tile, int V)
    {
        const Lane L = Tl::make_lane(tile * kTileV, V);
        Ctx X;
        init_tofs(X, L);
        f4 h[HR][T];
        f4 sv[T];
        Tl::load_state(sv, rsrc(S0c ? S0c : C.H, S0c ? L.state_bytes : 0u), L);
#pragma unroll
        for (int i = 0; i < HA; ++i) {
            const bool live = i < C.n_seg;
            Tl::load_state(h[i], rsrc(C.H + (size_t)sg(C, live ? i : 0) * (L.state_bytes / 4),
                                      live ? L.state_bytes : 0u), L);
        }
        Tl::frag_from_vecs(X.own, sv);
        Tl::put_state(lds, X.own, L);
        int s = 0;
        for (; s + HR <= C.n_seg; s += HR) {
            step<0>(s, X, C, h, lds, L);
            if constexpr (HR > 1) step<1 % HR>(s + 1, X, C, h, lds, L);
            if constexpr (HR > 2) step<2 % HR>(s + 2, X, C, h, lds, L);
            if constexpr (HR > 3) step<3 % HR>(s + 3, X, C, h, lds, L);
            if constexpr (HR > 4) step<4 % HR>(s + 4, X, C, h, lds, L);
        }
        tail<0>(s, X, C, h, lds, L);
        Tl::store_state(rsrc(C.out + (size_t)sg(C, C.n_seg - 1) * (L.state_bytes / 4), L.state_bytes), X.own,
                        L);
    }

    // One step of a group (G = 2), entered right after the barrier that opens
    // it: the stage and state reads, the first half of the MFMA blocks, the
    // mid-step barrier (the other group's step boundary; every read of this
    // group's state slot has returned before it, so the slot can then take
    // the new state), the second half with out of step s-1 and H of step
    // s+HA, the new state into the slot, and the barrier that closes the step
    // unless this is group 1's last step (group 1 ends one barrier after the
    // others' last).
    static constexpr int kMid = BP / 2;
    static constexpr int kS2 = kStoreAt > kMid ? kStoreAt : kMid;
    static constexpr int kL2 = kLoadAt > kS2 ? kLoadAt : kS2;
    template <int LSX>
    static __device__ __forceinline__ void step_pair(int s, int g, Ctx& X, const Chain& C, f4 (&h)[HR][T], float* lds,
                                                     float* slot, const Lane& L)
    {
        s = __builtin_amdgcn_readfirstlane(s);
        const int jp = s > 0 ? sg(C, s - 1) : 0;
        X.out_prev = rsrc(C.out + (size_t)jp * (L.state_bytes / 4), s > 0 ? L.state_bytes : 0u);
        const bool live = s + HA < C.n_seg;
        const __amdgpu_buffer_rsrc_t Hr =
            rsrc(C.H + (size_t)(live ? sg(C, s + HA) : 0) * (L.state_bytes / 4), live ? L.state_bytes : 0u);

        __builtin_amdgcn_sched_barrier(0);
        debug_delay(L.wave, s, 0);
        X.cur = slot;
        X.st = lds + S::STATE_FLOATS + (s & 1) * STAGE + (DIR == QLA_DIR_FWD ? L.a0 * K : 0);
#pragma unroll
        for (int b = 0; b < kFirstReads; ++b)
#pragma unroll
            for (int t = 0; t < T; ++t) X.mo[b][t] = rd(X.st, t, b, L, X.tofs);
        Tl::template read_pv<0, kOwn, BP>(X.pv, X.cur, L);
        {
            f4 hx[T];
            Tl::frag_from_vecs(hx, h[LSX]);
#pragma unroll
            for (int t = 0; t < T; ++t) X.acc[t] = hx[t];
        }
        __builtin_amdgcn_sched_barrier(0);
        blocks<0, kMid>(X, L);
        lds_handoff();
        // The second half: this group's step ends at the next barrier.  Its
        // waves take issue priority over the other group's (in the first half
        // of its step), so its MFMAs finish first and the other group's
        // remaining MFMAs keep the matrix cores busy while this group writes
        // its state and reaches the barrier.
        __builtin_amdgcn_s_setprio(1);
        blocks<kMid, kS2>(X, L);
        Tl::store_state(X.out_prev, X.own, L);
        __builtin_amdgcn_sched_barrier(0);
        blocks<kS2, kL2>(X, L);
        Tl::load_state(h[(LSX + HA) % HR], Hr, L);
        __builtin_amdgcn_sched_barrier(0);
        blocks<kL2, BP>(X, L);

        debug_delay(L.wave, s, 1);
        Tl::put_state(slot, X.acc, L);
#pragma unroll
        for (int t = 0; t < T; ++t) X.own[t] = X.acc[t];
        __builtin_amdgcn_sched_barrier(0);
        if (!(g == 1 && s + 1 == C.n_seg)) lds_handoff();
        __builtin_amdgcn_s_setprio(0);
    }

    template <int LSX>
    static __device__ __forceinline__ void tail_pair(int s, int g, Ctx& X, const Chain& C, f4 (&h)[HR][T],
                                                     float* lds, float* slot, const Lane& L)
    {
        if constexpr (LSX < HR - 1) {
            if (s + LSX < C.n_seg) {
                step_pair<LSX>(s + LSX, g, X, C, h, lds, slot, L);
                tail_pair<LSX + 1>(s, g, X, C, h, lds, slot, L);
            }
        }
    }

    static __device__ __forceinline__ void consumer_pair(const Chain& C, const float* S0c, float* lds, int tp,
                                                         int V)
    {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int g = wave / CWG;
        const int pairs = ((V + kTileV - 1) / kTileV + 1) / 2;
        const Lane L = Tl::make_lane((tp + g * pairs) * kTileV, V, K, wave - g * CWG);
        float* slot = lds + g * (kTileV * LS);  // the group's one state slot
        Ctx X;
        init_tofs(X, L);
        f4 h[HR][T];
        f4 sv[T];
        Tl::load_state(sv, rsrc(S0c ? S0c : C.H, S0c ? L.state_bytes : 0u), L);
#pragma unroll
        for (int i = 0; i < HA; ++i) {
            const bool live = i < C.n_seg;
            Tl::load_state(h[i], rsrc(C.H + (size_t)sg(C, live ? i : 0) * (L.state_bytes / 4),
                                      live ? L.state_bytes : 0u), L);
        }
        Tl::frag_from_vecs(X.own, sv);
        Tl::put_state(slot, X.own, L);
        lds_handoff();             // barrier 0: both initial states and M_0 in place
        if (g == 1) lds_handoff(); // barrier 1: group 1 starts half a step later
        int s = 0;
        for (; s + HR <= C.n_seg; s += HR) {
            step_pair<0>(s, g, X, C, h, lds, slot, L);
            if constexpr (HR > 1) step_pair<1 % HR>(s + 1, g, X, C, h, lds, slot, L);
            if constexpr (HR > 2) step_pair<2 % HR>(s + 2, g, X, C, h, lds, slot, L);
            if constexpr (HR > 3) step_pair<3 % HR>(s + 3, g, X, C, h, lds, slot, L);
            if constexpr (HR > 4) step_pair<4 % HR>(s + 4, g, X, C, h, lds, slot, L);
        }
        tail_pair<0>(s, g, X, C, h, lds, slot, L);
        Tl::store_state(rsrc(C.out + (size_t)sg(C, C.n_seg - 1) * (L.state_bytes / 4), L.state_bytes), X.own,
                        L);
    }

    static __device__ __forceinline__ void run(const float* H, const float* M, const float* S0, float* out,
                                               int n_seg, int V, size_t chain, int tile, float* lds)
    {
        const size_t state = (size_t)K * V;
        const Chain C{M + chain * (size_t)n_seg * K * K, H + chain * state * n_seg, out + chain * state * n_seg,
                      n_seg};
        run_chain(C, S0 ? S0 + chain * state : nullptr, V, tile, lds);
    }

    static __device__ __forceinline__ void run_chain(const Chain& C, const float* S0c, int V, int tile, float* lds)
    {
        // A chain without segments: every wave leaves before any barrier.
        if (__builtin_amdgcn_readfirstlane(C.n_seg) <= 0) return;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if constexpr (G == 1) {
            if (wave >= CW) producer(C, lds, wave - CW, tile, V);
            else consumer(C, S0c, lds, tile, V);
        } else {
            // tile: the pair index
            if (wave >= CW) producer_pair(C, lds, wave - CW, tile, V);
            else consumer_pair(C, S0c, lds, tile, V);
        }
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

// The general kernel: compute size 256, the caller's K in kp (PAD when kp < 256).
template <int LAYOUT, int DIR, bool PAD>
struct General {
    static constexpr int WAVES = general_waves(DIR == QLA_DIR_FWD);
    using Tl = Tile<256, LAYOUT, DIR, WAVES, PAD>;
};

template <int LAYOUT, int DIR, bool PAD>
__global__ __launch_bounds__(64 * general_waves(DIR == QLA_DIR_FWD)) void correct_h0_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int n_seg, int V, int tiles, int kp)
{
    using Tl = typename General<LAYOUT, DIR, PAD>::Tl;
    __shared__ __attribute__((aligned(16))) float lds[Tl::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    Tl::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds, kp);
}

template <int K>
constexpr int dma_threads()
{
    return 64 * (K / 16 + kProducers);
}

template <int K, int LAYOUT>
__global__ __launch_bounds__(dma_threads<K>()) void correct_h0_fwd_dma_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int n_seg, int V, int tiles)
{
    using D = DmaChain<K, LAYOUT>;
    __shared__ __attribute__((aligned(16))) float lds[D::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    D::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds);
}

// Two 16-column tiles of a chain per workgroup (tiles tp and tp + pairs), half
// a step apart (K a multiple of 32): plain calls for which use_pairs holds.
template <int K, int LAYOUT, int DIR>
__global__ __launch_bounds__(dma_threads<K>()) void correct_h0_pair_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int n_seg, int V, int pairs)
{
    using D = DmaChain<K, LAYOUT, DIR, 2>;
    __shared__ __attribute__((aligned(16))) float lds[D::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / pairs;
    const int tp = id - chain * pairs;
    D::run(H, M, S0, out, n_seg, V, (size_t)chain, tp, lds);
}

template <int K, int LAYOUT>
__global__ __launch_bounds__(dma_threads<K>()) void correct_h0_bwd_dma_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int n_seg, int V, int tiles)
{
    using D = DmaChain<K, LAYOUT, QLA_DIR_BWD>;
    __shared__ __attribute__((aligned(16))) float lds[D::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    D::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds);
}

// Variable-length chains: sequence b has offs[b+1] - offs[b] segments; its
// block of H / M / out starts at segment heads * offs[b] and holds its heads'
// chains back to back, so chain (b, h) starts at segment heads * offs[b] +
// h * n_b.  S0 is [n_seqs][heads][K][V] as usual; kk is the caller's K.
template <typename Chain>
__device__ __forceinline__ Chain varlen_chain(const float* H, const float* M, float* out, int heads, int V, int chain,
                                              const SeqTable& seqs, int kk)
{
    const int b = chain / heads, h = chain - b * heads;
    const int n = seqs.offs[b + 1] - seqs.offs[b];
    const size_t base = (size_t)heads * seqs.offs[b] + (size_t)h * n;  // in segments
    const size_t state = (size_t)kk * V;
    return Chain{M + base * kk * kk, H + base * state, out + base * state, n};
}

template <int LAYOUT, int DIR, bool PAD>
__global__ __launch_bounds__(64 * general_waves(DIR == QLA_DIR_FWD)) void correct_h0_varlen_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int heads, int V, int tiles, int kp,
    SeqTable seqs)
{
    using Tl = typename General<LAYOUT, DIR, PAD>::Tl;
    __shared__ __attribute__((aligned(16))) float lds[Tl::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    const int kk = PAD ? kp : 256;
    const auto C = varlen_chain<typename Tl::Chain>(H, M, out, heads, V, chain, seqs, kk);
    Tl::run_chain(C, S0 ? S0 + (size_t)chain * kk * V : nullptr, V, tile, lds, kp);
}

template <int K, int LAYOUT>
__global__ __launch_bounds__(dma_threads<K>()) void correct_h0_fwd_dma_varlen_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int heads, int V, int tiles,
    SeqTable seqs)
{
    using D = DmaChain<K, LAYOUT>;
    __shared__ __attribute__((aligned(16))) float lds[D::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    const auto C = varlen_chain<typename D::Chain>(H, M, out, heads, V, chain, seqs, K);
    D::run_chain(C, S0 ? S0 + (size_t)chain * K * V : nullptr, V, tile, lds);
}

// Variable-length chains with two tiles per workgroup (K a multiple of 32).
template <int K, int LAYOUT, int DIR>
__global__ __launch_bounds__(dma_threads<K>()) void correct_h0_pair_varlen_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int heads, int V, int pairs,
    SeqTable seqs)
{
    using D = DmaChain<K, LAYOUT, DIR, 2>;
    __shared__ __attribute__((aligned(16))) float lds[D::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / pairs;
    const int tp = id - chain * pairs;
    const auto C = varlen_chain<typename D::Chain>(H, M, out, heads, V, chain, seqs, K);
    D::run_chain(C, S0 ? S0 + (size_t)chain * K * V : nullptr, V, tp, lds);
}

template <int K, int LAYOUT>
__global__ __launch_bounds__(dma_threads<K>()) void correct_h0_bwd_dma_varlen_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int heads, int V, int tiles,
    SeqTable seqs)
{
    using D = DmaChain<K, LAYOUT, QLA_DIR_BWD>;
    __shared__ __attribute__((aligned(16))) float lds[D::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    const auto C = varlen_chain<typename D::Chain>(H, M, out, heads, V, chain, seqs, K);
    D::run_chain(C, S0 ? S0 + (size_t)chain * K * V : nullptr, V, tile, lds);
}

// Grouped calls.  K <= 128: one launch; each workgroup looks up its head's
// (layout, direction) and runs that variant of the producer kernel (every
// variant has the same block shape and LDS size there).
template <int K>
struct Grouped {
    static_assert(K <= 128, "one grouped launch covers the producer kernels");
    static constexpr int WAVES = K / 16 + kProducers;
    static constexpr int max2(int a, int b) { return a > b ? a : b; }
    static constexpr int LDS_FLOATS = max2(max2(DmaChain<K, QLA_LAYOUT_KV, QLA_DIR_FWD>::LDS_FLOATS,
                                                DmaChain<K, QLA_LAYOUT_KV, QLA_DIR_BWD>::LDS_FLOATS),
                                           max2(DmaChain<K, QLA_LAYOUT_VK, QLA_DIR_FWD>::LDS_FLOATS,
                                                DmaChain<K, QLA_LAYOUT_VK, QLA_DIR_BWD>::LDS_FLOATS));
};

template <int K>
constexpr int grouped_threads()
{
    return 64 * Grouped<K>::WAVES;
}

// The variant (2 * layout + direction) of the head group holding `head`.
__device__ __forceinline__ int group_variant(int head, const GroupTable& table)
{
    int variant = 0;
    for (int i = 0; i < table.n; ++i)
        if (head >= table.begin[i] && head < table.begin[i] + table.count[i]) variant = table.variant[i];
    return variant;
}

template <int K>
__global__ __launch_bounds__((grouped_threads<K>())) void correct_h0_grouped_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int n_seg, int V, int tiles, int heads,
    GroupTable table)
{
    __shared__ __attribute__((aligned(16))) float lds[Grouped<K>::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / tiles;
    const int tile = id - chain * tiles;
    switch (group_variant(chain % heads, table)) {
    case 0: DmaChain<K, QLA_LAYOUT_KV, QLA_DIR_FWD>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    case 1: DmaChain<K, QLA_LAYOUT_KV, QLA_DIR_BWD>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    case 2: DmaChain<K, QLA_LAYOUT_VK, QLA_DIR_FWD>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    default: DmaChain<K, QLA_LAYOUT_VK, QLA_DIR_BWD>::run(H, M, S0, out, n_seg, V, (size_t)chain, tile, lds); break;
    }
}

// The grouped call with two tiles of a chain per workgroup (K a multiple of
// 32), chosen by the same rule as for plain calls: each head group's chains
// run the plain calls' two-tile code for its variant.
template <int K>
__global__ __launch_bounds__((grouped_threads<K>())) void correct_h0_grouped_pair_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int n_seg, int V, int pairs, int heads,
    GroupTable table)
{
    static_assert(DmaChain<K, QLA_LAYOUT_KV, QLA_DIR_FWD, 2>::LDS_FLOATS <= Grouped<K>::LDS_FLOATS &&
                      DmaChain<K, QLA_LAYOUT_VK, QLA_DIR_BWD, 2>::LDS_FLOATS <= Grouped<K>::LDS_FLOATS,
                  "the two-tile chains fit the grouped LDS");
    __shared__ __attribute__((aligned(16))) float lds[Grouped<K>::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int chain = id / pairs;
    const int tp = id - chain * pairs;
    switch (group_variant(chain % heads, table)) {
    case 0: DmaChain<K, QLA_LAYOUT_KV, QLA_DIR_FWD, 2>::run(H, M, S0, out, n_seg, V, (size_t)chain, tp, lds); break;
    case 1: DmaChain<K, QLA_LAYOUT_KV, QLA_DIR_BWD, 2>::run(H, M, S0, out, n_seg, V, (size_t)chain, tp, lds); break;
    case 2: DmaChain<K, QLA_LAYOUT_VK, QLA_DIR_FWD, 2>::run(H, M, S0, out, n_seg, V, (size_t)chain, tp, lds); break;
    default: DmaChain<K, QLA_LAYOUT_VK, QLA_DIR_BWD, 2>::run(H, M, S0, out, n_seg, V, (size_t)chain, tp, lds); break;
    }
}

// K > 128: the general kernel's backward block (four waves, a whole 128-byte
// line per M row load) differs from its forward one (eight waves), so the
// groups of one direction run as one launch, the other direction's as a
// second.  `table` holds only this launch's groups, and the launch covers
// batch x sel chains, sel = the heads in those groups: logical chain c is
// batch entry c / sel and the (c % sel)-th head of the groups taken in table
// order.
template <int DIR, bool PAD>
struct GroupedDir {
    static constexpr int WAVES = general_waves(DIR == QLA_DIR_FWD);
    using TK = Tile<256, QLA_LAYOUT_KV, DIR, WAVES, PAD>;
    using TV = Tile<256, QLA_LAYOUT_VK, DIR, WAVES, PAD>;
    static constexpr int LDS_FLOATS = TK::LDS_FLOATS > TV::LDS_FLOATS ? TK::LDS_FLOATS : TV::LDS_FLOATS;
};

template <int DIR, bool PAD>
__global__ __launch_bounds__(64 * general_waves(DIR == QLA_DIR_FWD)) void correct_h0_grouped_dir_kernel(
    const float* H, const float* __restrict__ M, const float* S0, float* out, int n_seg, int V, int tiles, int heads,
    int kp, int sel, GroupTable table)
{
    using G = GroupedDir<DIR, PAD>;
    __shared__ __attribute__((aligned(16))) float lds[G::LDS_FLOATS];
    const int id = xcd_logical_id(blockIdx.x, gridDim.x);
    const int c = id / tiles;
    const int tile = id - c * tiles;
    const int b = c / sel;
    int j = c - b * sel;
    int head = 0, layout = QLA_LAYOUT_KV;
    for (int i = 0; i < table.n; ++i) {
        if (j >= 0 && j < table.count[i]) {
            head = table.begin[i] + j;
            layout = table.variant[i] >> 1;
        }
        j -= table.count[i];
    }
    const size_t chain = (size_t)b * heads + head;
    if (layout == QLA_LAYOUT_KV) G::TK::run(H, M, S0, out, n_seg, V, chain, tile, lds, kp);
    else G::TV::run(H, M, S0, out, n_seg, V, chain, tile, lds, kp);
}

// ---- launchers ------------------------------------------------------------
template <int K, int LAYOUT, int DIR>
hipError_t launch_dma(const LaunchArgs& a, dim3 grid, int tiles)
{
    if constexpr (DIR == QLA_DIR_FWD)
        hipLaunchKernelGGL((correct_h0_fwd_dma_kernel<K, LAYOUT>), grid, dim3(dma_threads<K>()), 0,
                           (hipStream_t)a.stream, a.H, a.M, a.S0, a.out, a.n_seg, a.V, tiles);
    else
        hipLaunchKernelGGL((correct_h0_bwd_dma_kernel<K, LAYOUT>), grid, dim3(dma_threads<K>()), 0,
                           (hipStream_t)a.stream, a.H, a.M, a.S0, a.out, a.n_seg, a.V, tiles);
    return hipGetLastError();
}

template <int K, int LAYOUT, int DIR>
hipError_t launch_dma_varlen(const LaunchArgs& a, dim3 grid, int tiles, const SeqTable& seqs)
{
    if constexpr (DIR == QLA_DIR_FWD)
        hipLaunchKernelGGL((correct_h0_fwd_dma_varlen_kernel<K, LAYOUT>), grid, dim3(dma_threads<K>()), 0,
                           (hipStream_t)a.stream, a.H, a.M, a.S0, a.out, a.heads, a.V, tiles, seqs);
    else
        hipLaunchKernelGGL((correct_h0_bwd_dma_varlen_kernel<K, LAYOUT>), grid, dim3(dma_threads<K>()), 0,
                           (hipStream_t)a.stream, a.H, a.M, a.S0, a.out, a.heads, a.V, tiles, seqs);
    return hipGetLastError();
}

// The groups of direction DIR of a grouped call at K > 128, as one launch
// (none if the call has no such group).
template <int DIR, bool PAD>
hipError_t launch_grouped_dir(const LaunchArgs& a, int tiles, const GroupTable& all)
{
    GroupTable t{};
    int sel = 0;
    for (int i = 0; i < all.n; ++i) {
        if ((all.variant[i] & 1) != DIR) continue;
        t.begin[t.n] = all.begin[i];
        t.count[t.n] = all.count[i];
        t.variant[t.n] = all.variant[i];
        sel += all.count[i];
        ++t.n;
    }
    if (sel == 0) return hipSuccess;
    const long long batch = a.chains / a.heads;
    const dim3 grid((unsigned)(batch * sel * tiles));
    hipLaunchKernelGGL((correct_h0_grouped_dir_kernel<DIR, PAD>), grid, dim3(64 * general_waves(DIR == QLA_DIR_FWD)),
                       0, (hipStream_t)a.stream, a.H, a.M, a.S0, a.out, a.n_seg, a.V, tiles, a.heads, a.K, sel, t);
    return hipGetLastError();
}

// Whether a plain call runs two tiles per workgroup (measured on 256 CUs, 8
// to 64 segments).  At K >= 96 one workgroup fits in a CU's LDS with either
// kernel, so a call runs in rounds of `cus` workgroups, and a two-tile
// workgroup takes 1.7-2.0x as long as a one-tile one: pairs pay off when they
// save enough rounds, 1.8 r2 < r1 (at 1-2 tiles per CU one round against two,
// at 3-4 two against four; at 2-3 tiles per CU two rounds of pairs lose to
// three of single tiles).  Below K = 96 several workgroups share a CU: single
// tiles win up to three tiles per CU and pairs at three to four; beyond four
// the two are within 10% either way, and pairs are kept at K = 32, where they
// win more often.  At K = 64 chains of 32 or more segments gain from pairs at
// 1-2 tiles per CU as well.
template <int K>
bool use_pairs(long long chains, int tiles, int n_seg, int cus)
{
    const long long t1 = chains * tiles, t2 = chains * ((tiles + 1) / 2);
    if constexpr (K >= 96) {
        const long long r1 = (t1 + cus - 1) / cus, r2 = (t2 + cus - 1) / cus;
        return 9 * r2 < 5 * r1;
    } else {
        if (K == 64 && n_seg >= 32 && t1 > cus && t1 <= 2LL * cus) return true;
        return t1 > 3LL * cus && (K != 64 || t1 <= 4LL * cus);
    }
}

// Mean segments per sequence of a variable-length call.
inline int mean_segments(const SeqTable& seqs)
{
    return seqs.n > 0 ? (seqs.offs[seqs.n] - seqs.offs[0]) / seqs.n : 0;
}

// kind: 0 plain, 1 variable-length, 2 grouped.
template <int K, int LAYOUT, int DIR>
hipError_t launch_k(const LaunchArgs& a, int kind, const SeqTable* seqs, const GroupTable* table)
{
    const int tiles = (a.V + kTileV - 1) / kTileV;
    const dim3 grid((unsigned)(a.chains * tiles));
    if constexpr (K <= 128) {
        if (kind == 2) {
            if constexpr (K % 32 == 0) {
                if (tiles >= 2 && use_pairs<K>(a.chains, tiles, a.n_seg, a.cus)) {
                    const int pairs = (tiles + 1) / 2;
                    hipLaunchKernelGGL((correct_h0_grouped_pair_kernel<K>), dim3((unsigned)(a.chains * pairs)),
                                       dim3(grouped_threads<K>()), 0, (hipStream_t)a.stream, a.H, a.M, a.S0, a.out,
                                       a.n_seg, a.V, pairs, a.heads, *table);
                    return hipGetLastError();
                }
            }
            hipLaunchKernelGGL((correct_h0_grouped_kernel<K>), grid, dim3(grouped_threads<K>()), 0,
                               (hipStream_t)a.stream, a.H, a.M, a.S0, a.out, a.n_seg, a.V, tiles, a.heads, *table);
            return hipGetLastError();
        }
        if constexpr (K % 32 == 0) {
            // Pairs of tiles, half a step apart, so that one tile's step
            // boundary overlaps the other's matrix work (variable-length
            // calls: judged by their mean chain length).
            const int n = kind == 1 ? mean_segments(*seqs) : a.n_seg;
            if (tiles >= 2 && use_pairs<K>(a.chains, tiles, n, a.cus)) {
                const int pairs = (tiles + 1) / 2;
                const dim3 pgrid((unsigned)(a.chains * pairs));
                if (kind == 1)
                    hipLaunchKernelGGL((correct_h0_pair_varlen_kernel<K, LAYOUT, DIR>), pgrid, dim3(dma_threads<K>()),
                                       0, (hipStream_t)a.stream, a.H, a.M, a.S0, a.out, a.heads, a.V, pairs, *seqs);
                else
                    hipLaunchKernelGGL((correct_h0_pair_kernel<K, LAYOUT, DIR>), pgrid, dim3(dma_threads<K>()), 0,
                                       (hipStream_t)a.stream, a.H, a.M, a.S0, a.out, a.n_seg, a.V, pairs);
                return hipGetLastError();
            }
        }
        return kind == 1 ? launch_dma_varlen<K, LAYOUT, DIR>(a, grid, tiles, *seqs)
                         : launch_dma<K, LAYOUT, DIR>(a, grid, tiles);
    } else {
        // K == 256: exact; 128 < a.K < 256: zero-padded to 256.
        constexpr bool PAD = K != 256;
        const int threads = 64 * general_waves(DIR == QLA_DIR_FWD);
        if (kind == 2) {
            hipError_t e = launch_grouped_dir<QLA_DIR_FWD, PAD>(a, tiles, *table);
            return e != hipSuccess ? e : launch_grouped_dir<QLA_DIR_BWD, PAD>(a, tiles, *table);
        } else if (kind == 1) {
            hipLaunchKernelGGL((correct_h0_varlen_kernel<LAYOUT, DIR, PAD>), grid, dim3(threads), 0,
                               (hipStream_t)a.stream, a.H, a.M, a.S0, a.out, a.heads, a.V, tiles, a.K, *seqs);
        } else {
            hipLaunchKernelGGL((correct_h0_kernel<LAYOUT, DIR, PAD>), grid, dim3(threads), 0, (hipStream_t)a.stream,
                               a.H, a.M, a.S0, a.out, a.n_seg, a.V, tiles, a.K);
        }
        return hipGetLastError();
    }
}

template <int K>
hipError_t launch_layout_dir(const LaunchArgs& a, int layout, int direction, int kind, const SeqTable* seqs,
                             const GroupTable* table)
{
    if (layout == QLA_LAYOUT_KV)
        return direction == QLA_DIR_FWD ? launch_k<K, QLA_LAYOUT_KV, QLA_DIR_FWD>(a, kind, seqs, table)
                                        : launch_k<K, QLA_LAYOUT_KV, QLA_DIR_BWD>(a, kind, seqs, table);
    return direction == QLA_DIR_FWD ? launch_k<K, QLA_LAYOUT_VK, QLA_DIR_FWD>(a, kind, seqs, table)
                                    : launch_k<K, QLA_LAYOUT_VK, QLA_DIR_BWD>(a, kind, seqs, table);
}

// The compiled kernel family for the caller's K (a multiple of 16 in [16, 256]).
hipError_t dispatch(const LaunchArgs& a, int layout, int direction, int kind, const SeqTable* seqs,
                    const GroupTable* table)
{
    switch (a.K) {
    case 16: return launch_layout_dir<16>(a, layout, direction, kind, seqs, table);
    case 32: return launch_layout_dir<32>(a, layout, direction, kind, seqs, table);
    case 48: return launch_layout_dir<48>(a, layout, direction, kind, seqs, table);
    case 64: return launch_layout_dir<64>(a, layout, direction, kind, seqs, table);
    case 80: return launch_layout_dir<80>(a, layout, direction, kind, seqs, table);
    case 96: return launch_layout_dir<96>(a, layout, direction, kind, seqs, table);
    case 112: return launch_layout_dir<112>(a, layout, direction, kind, seqs, table);
    case 128: return launch_layout_dir<128>(a, layout, direction, kind, seqs, table);
    case 256: return launch_layout_dir<256>(a, layout, direction, kind, seqs, table);
    default:
        if (a.K > 128 && a.K < 256 && a.K % 16 == 0) return launch_layout_dir<255>(a, layout, direction, kind, seqs, table);
        return hipErrorInvalidValue;
    }
}

}  // namespace

int tiles_for(int V) { return (V + kTileV - 1) / kTileV; }

bool plain_call_pairs_tiles(int K, long long chains, int V, int n_seg, int cus)
{
    const int tiles = tiles_for(V);
    if (tiles < 2) return false;
    switch (K) {
    case 32: return use_pairs<32>(chains, tiles, n_seg, cus);
    case 64: return use_pairs<64>(chains, tiles, n_seg, cus);
    case 96: return use_pairs<96>(chains, tiles, n_seg, cus);
    case 128: return use_pairs<128>(chains, tiles, n_seg, cus);
    default: return false;
    }
}

int max_threads_per_group() { return dma_threads<128>() > 64 * general_waves(true) ? dma_threads<128>() : 64 * general_waves(true); }

hipError_t launch_correct_h0(const LaunchArgs& a)
{
    return dispatch(a, a.layout, a.direction, 0, nullptr, nullptr);
}

hipError_t launch_correct_h0_varlen(const LaunchArgs& a, const SeqTable& seqs)
{
    return dispatch(a, a.layout, a.direction, 1, &seqs, nullptr);
}

hipError_t launch_correct_h0_grouped(const LaunchArgs& a, const GroupTable& table)
{
    // The variant is chosen per head inside the kernel; layout/direction here
    // only select a template instance, which the grouped launch ignores.
    return dispatch(a, QLA_LAYOUT_KV, QLA_DIR_FWD, 2, nullptr, &table);
}

}  // namespace qla
