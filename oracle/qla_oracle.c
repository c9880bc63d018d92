/*
 * qla_oracle.c -- plain fp64 CPU oracle for the context-parallel (CP)
 * state-correction recurrence.  TEST INFRASTRUCTURE ONLY: tests, the smoke
 * check and the CPU-baseline leg of the benchmark call it; the product path
 * never does.  It shares no code, header or constant with the HIP library.
 *
 * Source (cited by title and section):
 *   Antarx Memos, "一次 TileLang Warp Specialization 数值错误的定位与修复：
 *   从双缓冲竞争到 membar" (the FlashQLA correction note).
 *   - section "从版本升级后的数值偏差开始" (the deviation after the upgrade):
 *     one routine does both the forward initial-state correction and the
 *     backward terminal-state correction of CP; the state is stored either as
 *     kv (K x V) or as vk (V x K), and the layout decides on which side the
 *     multiply happens and where the transposes go.
 *   - section "理解三个缓冲区，才能判断哪里需要同步" (the three buffers):
 *     H_i is the segment-local state, M_i the propagation matrix, and the
 *     corrected state is propagate(M_i, previous state) plus H_i, where
 *     propagate picks the product by layout and direction.  The printed
 *     formula was lost in extraction; the form used here is the plain one:
 *       forward : S_i = M_i   * S_{i-1} + H_i,  i = 0 .. n-1
 *       backward: G_i = M_i^T * G_{i+1} + H_i,  i = n-1 .. 0
 *     written for the K x V (kv) view; the vk layout stores the transpose and
 *     therefore multiplies on the right (S_vk * M^T forward, S_vk * M
 *     backward).  S_{-1} / G_n is the optional initial state S0 (absent =
 *     zero).  Both directions pair M[j] with H[j] to produce out[j].
 *   - section "决定性证据：错误值来自同一槽位的下一代": the backward pass walks
 *     the segments in reverse order.
 *
 * Arithmetic: every product and sum in fp64, the contraction index ascending,
 * no blocking and no reordering.  Inputs are fp64 (callers upcast the exact
 * fp32 values the GPU receives); outputs are fp64, not rounded.
 *
 * Array shapes (C order, dense):
 *   H, out : [chains][n_seg][K][V] (kv)  or  [chains][n_seg][V][K] (vk)
 *   M      : [chains][n_seg][K][K]       (same array for both layouts)
 *   S0     : [chains][K][V] (kv) or [chains][V][K] (vk), or NULL (= zero)
 */
#include <stdlib.h>
#include <string.h>

#define ORACLE_KV 0
#define ORACLE_VK 1
#define ORACLE_FWD 0
#define ORACLE_BWD 1

/* Element (a, b) of the operator applied in one step: M itself forward, its
 * transpose backward. */
static double op_elem(const double* Mj, int K, int direction, int a, int b)
{
    return direction == ORACLE_FWD ? Mj[(size_t)a * K + b] : Mj[(size_t)b * K + a];
}

/* propagate for the kv layout: Y[a][v] = sum_b op(a,b) * S[b][v]. */
static void propagate_kv(const double* Mj, const double* S, double* Y,
                         int K, int V, int direction)
{
    for (int a = 0; a < K; ++a)
        for (int v = 0; v < V; ++v) {
            double acc = 0.0;
            for (int b = 0; b < K; ++b)
                acc += op_elem(Mj, K, direction, a, b) * S[(size_t)b * V + v];
            Y[(size_t)a * V + v] = acc;
        }
}

/* propagate for the vk layout: the state is stored transposed (V x K), so the
 * operator multiplies from the right: Y[v][a] = sum_b S[v][b] * op(a,b). */
static void propagate_vk(const double* Mj, const double* S, double* Y,
                         int K, int V, int direction)
{
    for (int v = 0; v < V; ++v)
        for (int a = 0; a < K; ++a) {
            double acc = 0.0;
            for (int b = 0; b < K; ++b)
                acc += S[(size_t)v * K + b] * op_elem(Mj, K, direction, a, b);
            Y[(size_t)v * K + a] = acc;
        }
}

/* Returns 0 on success, -1 on a bad argument, -2 if scratch allocation fails. */
int qla_oracle_correct_h0(const double* H, const double* M, const double* S0,
                          double* out, int layout, int direction,
                          long chains, int n_seg, int K, int V)
{
    if (!H || !M || !out) return -1;
    if (layout != ORACLE_KV && layout != ORACLE_VK) return -1;
    if (direction != ORACLE_FWD && direction != ORACLE_BWD) return -1;
    if (chains < 0 || n_seg < 0 || K < 1 || V < 1) return -1;

    const size_t state = (size_t)K * V;
    const size_t mat = (size_t)K * K;
    double* S = (double*)malloc(state * sizeof(double));
    double* Y = (double*)malloc(state * sizeof(double));
    if (!S || !Y) { free(S); free(Y); return -2; }

    for (long c = 0; c < chains; ++c) {
        /* Chain start: S0 if given, zero otherwise. */
        if (S0) memcpy(S, S0 + (size_t)c * state, state * sizeof(double));
        else memset(S, 0, state * sizeof(double));

        for (int s = 0; s < n_seg; ++s) {
            const int j = direction == ORACLE_FWD ? s : n_seg - 1 - s;
            const double* Mj = M + ((size_t)c * n_seg + j) * mat;
            const double* Hj = H + ((size_t)c * n_seg + j) * state;
            double* Oj = out + ((size_t)c * n_seg + j) * state;

            if (layout == ORACLE_KV) propagate_kv(Mj, S, Y, K, V, direction);
            else propagate_vk(Mj, S, Y, K, V, direction);

            for (size_t e = 0; e < state; ++e) S[e] = Y[e] + Hj[e];
            memcpy(Oj, S, state * sizeof(double));
        }
    }
    free(S);
    free(Y);
    return 0;
}
