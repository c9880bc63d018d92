/*
 * qla.h -- C ABI of the MI355X (gfx950) context-parallel state-correction
 * library (libqla.so).
 *
 * The operation (Antarx Memos, "一次 TileLang Warp Specialization 数值错误的
 * 定位与修复：从双缓冲竞争到 membar", the FlashQLA correction note):
 *   - section "从版本升级后的数值偏差开始": under context parallelism a long
 *     sequence is cut into segments; each segment's local result is later
 *     combined with the state carried across segments.  One routine performs
 *     both the forward initial-state correction and the backward
 *     terminal-state correction.  The state is kept either as kv (K x V) or
 *     as vk (V x K); the layout changes the side of the product and the
 *     transposes.
 *   - section "理解三个缓冲区，才能判断哪里需要同步": H_i is a segment's local
 *     state, M_i its propagation matrix, and the corrected state is the
 *     previous state propagated through M_i plus H_i.
 *   - section "决定性证据：错误值来自同一槽位的下一代": the backward pass walks
 *     the segments in reverse order.
 *
 * In the kv view (X = S for kv, X = S^T for vk), per chain:
 *   forward : P = X(S0) (0 if S0 is NULL); for j = 0 .. n_seg-1:
 *             P = M[j]   * P + X(H[j]);  out[j] = P
 *   backward: P = X(S0) (0 if S0 is NULL); for j = n_seg-1 .. 0:
 *             P = M[j]^T * P + X(H[j]);  out[j] = P
 * For vk this is S[j] = S[j-1] * M[j]^T + H[j] (forward) and
 * S[j] = S[j+1] * M[j] + H[j] (backward) on the stored V x K matrices.
 * Arithmetic is fp32 throughout (fp32 products, fp32 accumulation on the
 * matrix cores, no reduced-precision inputs).  Results are deterministic:
 * identical inputs give bit-identical outputs on every call.
 *
 * Memory (all device pointers, fp32, dense, C order, 16-byte aligned):
 *   H, out : [batch][heads][n_seg][K][V] (kv)  or  [batch][heads][n_seg][V][K] (vk)
 *   M      : [batch][heads][n_seg][K][K]       (one array for both layouts)
 *   S0     : [batch][heads][K][V] (kv) or [batch][heads][V][K] (vk), or NULL
 * Ownership: the caller allocates and frees every buffer; the library
 * allocates nothing, keeps no mutable global state, never synchronises and
 * never prints.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns.  Every element of out is written.  out may be
 * the same pointer as H (in place); any other overlap of out with H, M or S0
 * is rejected.
 *
 * Errors: arguments are checked before anything is enqueued and a negative
 * status is returned without launching.  A launch failure reported by the
 * runtime returns QLA_ERR_LAUNCH.  Faults inside the kernel surface at the
 * caller's next synchronisation on the stream.
 */
#ifndef QLA_H
#define QLA_H

#ifdef __cplusplus
extern "C" {
#endif

#define QLA_API __attribute__((visibility("default")))

/* State layouts (correction note, section on the deviation after the upgrade). */
#define QLA_LAYOUT_KV 0 /* state stored K x V */
#define QLA_LAYOUT_VK 1 /* state stored V x K */

/* Directions: forward initial-state / backward terminal-state correction. */
#define QLA_DIR_FWD 0
#define QLA_DIR_BWD 1

/* Status codes. */
#define QLA_OK 0
#define QLA_ERR_NULL (-1)   /* H, M or out is NULL */
#define QLA_ERR_ENUM (-2)   /* layout or direction not one of the values above */
#define QLA_ERR_SHAPE (-3)  /* K not a multiple of 16 in [16, 256], V not a multiple
                               of 4 in [4, 4096], a negative count, or a size that
                               overflows the launch limits */
#define QLA_ERR_ALIGN (-4)  /* a pointer not 16-byte aligned */
#define QLA_ERR_ALIAS (-5)  /* out overlaps H (other than out == H), M or S0 */
#define QLA_ERR_GROUPS (-6) /* head groups do not partition [0, heads) */
#define QLA_ERR_LAUNCH (-7) /* the runtime rejected the launch */
#define QLA_ERR_MEMORY (-8) /* a pointer is not device memory, or the extent the
                               call needs runs past the end of its allocation */
#define QLA_ERR_SEQS (-9)   /* segment offsets of a variable-length call: NULL, more
                               than QLA_MAX_SEQS sequences, not starting at 0, or
                               decreasing */

/* Largest number of head groups one grouped call accepts. */
#define QLA_MAX_GROUPS 64

/* Largest number of sequences one variable-length call accepts. */
#define QLA_MAX_SEQS 256

/* One head group of a grouped call: heads [head_begin, head_begin+head_count)
 * of every batch entry use this layout and direction. */
typedef struct {
    int head_begin;
    int head_count;
    int layout;    /* QLA_LAYOUT_KV or QLA_LAYOUT_VK */
    int direction; /* QLA_DIR_FWD or QLA_DIR_BWD */
} qla_head_group;

/*
 * qla_correct_h0 -- correct the segment states of batch*heads independent
 * chains, all with the same layout and direction.
 *   H, M, S0, out : device pointers as described above; S0 may be NULL.
 *   layout        : QLA_LAYOUT_KV or QLA_LAYOUT_VK.
 *   direction     : QLA_DIR_FWD or QLA_DIR_BWD.
 *   batch, heads  : chain grid (>= 0; a zero count, or n_seg == 0, is an empty
 *                   call that returns QLA_OK and enqueues nothing).
 *   n_seg         : segments per chain (>= 0).
 *   K             : key dimension (size of M), a multiple of 16 in [16, 256].
 *   V             : value dimension, a multiple of 4 in [4, 4096].
 *   stream        : hipStream_t to enqueue on.
 * Returns QLA_OK or a QLA_ERR_* code.
 */
QLA_API int qla_correct_h0(const float* H, const float* M, const float* S0, float* out,
                   int layout, int direction, int batch, int heads, int n_seg,
                   int K, int V, void* stream);

/*
 * qla_correct_h0_grouped -- one call over batch*heads chains whose layout and
 * direction vary by head group: one launch at K <= 128; above, the forward
 * groups and the backward groups are one launch each (the two directions use
 * different block shapes there), both enqueued on `stream`.  `groups` is a HOST array of n_groups entries
 * (1 <= n_groups <= QLA_MAX_GROUPS) whose head ranges must partition
 * [0, heads) exactly; it is copied into the launch and may be freed on return.
 * Buffers are laid out as for qla_correct_h0, with each head's matrices in its
 * own group's layout (K x V or V x K); a head occupies n_seg*K*V floats of H
 * and out and K*V floats of S0 either way.  Other arguments and the return
 * value are as for qla_correct_h0.
 */
QLA_API int qla_correct_h0_grouped(const float* H, const float* M, const float* S0, float* out,
                           const qla_head_group* groups, int n_groups,
                           int batch, int heads, int n_seg, int K, int V, void* stream);

/*
 * qla_correct_h0_varlen -- like qla_correct_h0 for n_seqs sequences whose
 * segment counts differ (the correction note, section "性能结果", benchmarks the
 * operator on variable-length inputs).  Sequence b has
 * n_b = seg_offsets[b+1] - seg_offsets[b] segments (n_b >= 0) and `heads`
 * chains.
 *   seg_offsets : HOST array of n_seqs + 1 ints, seg_offsets[0] = 0,
 *                 non-decreasing; copied into the launch, may be freed on
 *                 return.  0 <= n_seqs <= QLA_MAX_SEQS.
 *   H, out      : sequences back to back, sequence b's block starting at
 *                 segment heads * seg_offsets[b] (i.e. at float
 *                 heads * seg_offsets[b] * K * V) and laid out
 *                 [heads][n_b][K][V] (kv) or [heads][n_b][V][K] (vk); in
 *                 total heads * seg_offsets[n_seqs] segment states.
 *   M           : the same with K x K matrices.
 *   S0          : [n_seqs][heads][K][V] (kv) or [..][V][K] (vk), or NULL.
 * With every n_b equal to n this is exactly qla_correct_h0 with batch =
 * n_seqs and n_seg = n.  A sequence with n_b = 0 writes nothing (its S0
 * may still be read);
 * a call with no segments at all is an empty call (QLA_OK, nothing
 * enqueued).  Bad offsets return QLA_ERR_SEQS; other arguments, checks and
 * the return value are as for qla_correct_h0.
 */
QLA_API int qla_correct_h0_varlen(const float* H, const float* M, const float* S0, float* out,
                          int layout, int direction, const int* seg_offsets, int n_seqs,
                          int heads, int K, int V, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
QLA_API const char* qla_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLA_H */
