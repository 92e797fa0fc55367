/*
 * lisa.h -- C ABI of the MI355X (gfx950) LiSA forward-pass library, liblisa.so.
 *
 * LiSA (Linear Stochastic Attention) is described by the reading note
 * "LiSA:面向长程视觉建模的线性随机注意力" of arXiv:2611.04216v2; sections below
 * are that note's.  Per (batch, head) slice with n = grid_h * grid_w tokens in
 * row-major grid order (token i = row * grid_w + col):
 *
 *   global branch  [note §2.1-§2.3]
 *     phi = ReLU (or ELU + 1, lisa_problem.feature; the note's
 *     supplementary comparison of the two, Table 8);
 *     s = sum_j phi(K_j);  r_i = 1 / (phi(Q_i) . s + eps)
 *     Qt = diag(r) phi(Q);  S = Qt phi(K)^T   (row-stochastic up to eps)
 *     G  = sum_{k=0}^{T-1} diag(w_k) S^k V,  S^0 = I,
 *     computed as S^k V = Qt M^(k-1) (phi(K)^T V) with M = phi(K)^T Qt
 *     (Eq. 8), never forming an n x n matrix.
 *   step weights  [note §2.2 Eq. 4; §2.4 Eq. 10]
 *     geometric: w_k = (1-beta) beta^k / (1-beta^T), the same for every token;
 *     adaptive : w_k(i) given per token and head, used as given.
 *   local branch  [note §2.4, Fig. 2]
 *     L_i = sum_{j in N(i)} e_ij V_j / sum_{j in N(i)} e_ij,
 *     e_ij = exp(Q_i . K_j / sqrt(d_h)), N(i) = token i and its spatial
 *     neighbours in the 3x3 window, clipped at the grid border.  Q and K are
 *     used as given (no feature map) in this branch.
 *   mix  [note §2.4; §4.4 Table 6]
 *     Y = alpha_h G + (1 - alpha_h) L, one alpha per head.
 *
 * Conventions for every entry point:
 *   - Array pointers are DEVICE pointers unless stated; the caller owns every
 *     buffer.  The library never allocates, frees or synchronises; work is
 *     enqueued on `stream` (a hipStream_t, NULL = the null stream) and the
 *     call returns at once.
 *   - Q, K: [batch, heads, n, d_h]; V: [batch, heads, n, d_v]; Y: like V.
 *     Contiguous, element type `dtype`, 16-byte aligned.  Y must not overlap
 *     Q, K, V or the workspace.
 *   - Arguments are checked on the host before anything is enqueued; an
 *     error status means nothing was enqueued and nothing was written.  A
 *     failed launch is reported as LISA_ERR_HIP.  No C++ exception crosses
 *     the ABI.  NaN/Inf inputs are not checked; they propagate.
 *   - Workspace: `lisa_workspace_size` bytes of device memory, 256-byte
 *     aligned, ZERO-FILLED before its first use.  Every completed call leaves
 *     its counter words at zero again, so a workspace can be reused by later
 *     calls of any problem that fits it.  Calls that share a workspace must
 *     be ordered on one stream; concurrent calls on one workspace race.
 *   - Scheduling: a call launches one workgroup per compute unit, and groups
 *     of its workgroups (up to 256, as many as the problem splits a
 *     (batch, head) slice into) wait for each other.  The streaming kernel
 *     hands out ranks in the order workgroups start; the resident kernel
 *     gives a group consecutive workgroups (of one XCD where the group fits
 *     in one), which the device starts in order.  Either way a call
 *     completes when it can eventually run one group at a time (for the
 *     resident kernel, on one XCD); work on other streams only delays it.  A wait that lasts more than about half a second is abandoned (the
 *     call then finishes with undefined Y); that only happens if other work keeps a group's
 *     workgroups from starting for that long.  The call cannot report it when
 *     it returns (the work is asynchronous); it raises a flag in the
 *     workspace, which lisa_workspace_check reads and clears.
 *   - Arithmetic: fp32 accumulation throughout.  With LISA_BF16 inputs the
 *     matrix products run on bf16 MFMA with fp32 accumulation, and the
 *     operands the library derives itself (r_i phi(Q_i), powers of M applied
 *     to phi(Q_i), and the d_h x d_h statistics) are rounded to bf16 before
 *     entering a product; with LISA_FP32 inputs every product is fp32.
 *     Y is written in the input dtype (bf16: round to nearest even).
 */
#ifndef LISA_H
#define LISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lisa_status {
  LISA_OK = 0,
  LISA_ERR_NULL = 1,        /* a required pointer is NULL */
  LISA_ERR_SHAPE = 2,       /* a dimension is <= 0 or too large */
  LISA_ERR_PARAM = 3,       /* T outside 1..16 (1..8 with the predictor and the backward),
                               beta outside [0,1), eps <= 0 or not finite */
  LISA_ERR_DTYPE = 4,       /* dtype is not LISA_FP32 / LISA_BF16 */
  LISA_ERR_UNSUPPORTED = 5, /* d_h or d_v other than 64, or batch*heads > 65535 */
  LISA_ERR_WORKSPACE = 6,   /* workspace NULL, too small or not 256-byte aligned */
  LISA_ERR_ALIGN = 7,       /* Q, K, V, Y not 16-byte or weights/alpha/outputs not 4-byte aligned */
  LISA_ERR_HIP = 8,         /* a HIP launch or copy failed */
  LISA_ERR_STALLED = 9,     /* a call abandoned a wait: its outputs are undefined (lisa_workspace_check) */
  LISA_ERR_SCRATCH = 10     /* the problem does not fit lisa_forward_noalloc's fixed scratch */
} lisa_status;

typedef enum lisa_dtype { LISA_FP32 = 0, LISA_BF16 = 1 } lisa_dtype;

/* Feature map phi of the global branch: ReLU(x), or ELU(x) + 1 (x + 1 above
 * zero, e^x at or below; positive, so S stays row-stochastic).  With bf16
 * inputs the ELU features are rounded to bf16 before the products, as the
 * inputs are. */
typedef enum lisa_feature { LISA_FEATURE_RELU = 0, LISA_FEATURE_ELU = 1 } lisa_feature;

/* Which forward kernel runs the pass.  Both compute the same quantities in
 * the same precision; they differ in schedule and so in the order of the
 * fp32 sums over tokens.
 *   AUTO      : the library's choice for the problem and device (zero): the
 *               resident kernel wherever it applies, else the streaming one.
 *   STREAMING : workgroups stream tiles through LDS in three passes over K
 *               (statistics, then the rescaled keys, then the output).
 *   RESIDENT  : each workgroup holds its tile of Q, K, V on chip for the
 *               whole pass (bf16 ReLU problems with T <= 8 whose tiles fit
 *               a workgroup); LISA_ERR_UNSUPPORTED where it does not apply.
 * lisa_forward, lisa_reduce, lisa_apply, lisa_forward_mlp and the backward's
 * statistics of one problem (same struct, same device) take the same kernel
 * and so form the same sums. */
typedef enum lisa_schedule {
  LISA_SCHEDULE_AUTO = 0,
  LISA_SCHEDULE_STREAMING = 1,
  LISA_SCHEDULE_RESIDENT = 2
} lisa_schedule;

/* Problem description.  n = grid_h * grid_w tokens per (batch, head). */
typedef struct lisa_problem {
  int32_t batch;  /* B >= 1 */
  int32_t heads;  /* >= 1; batch * heads <= 65535 */
  int32_t grid_h; /* H >= 1 */
  int32_t grid_w; /* W >= 1; H * W <= 2^24 */
  int32_t d_h;    /* query/key width: 64 */
  int32_t d_v;    /* value width: 64 */
  int32_t T;      /* walk terms k = 0..T-1, 1 <= T <= 16; at most 8 for
                     lisa_forward_mlp and the backward entry points */
  int32_t dtype;  /* lisa_dtype of Q, K, V, Y */
  float eps;      /* row-normaliser stabiliser, finite and > 0 */
  int32_t feature; /* lisa_feature (0, ReLU, when zero-initialised); another
                      value: LISA_ERR_PARAM; ELU with lisa_forward_mlp or the
                      backward entry points: LISA_ERR_UNSUPPORTED */
  int32_t schedule; /* lisa_schedule (AUTO when zero-initialised); another
                       value: LISA_ERR_PARAM */
} lisa_problem;

/* Bytes of device workspace the calls below need for problem *p; 0 if *p is
 * invalid (or p is NULL).  Host only; enqueues nothing. */
size_t lisa_workspace_size(const lisa_problem* p);

/* The kernel lisa_forward runs for *p on the current device:
 * *schedule = LISA_SCHEDULE_STREAMING or LISA_SCHEDULE_RESIDENT (p->schedule
 * resolved; AUTO depends on the device's compute units).  Status as the
 * forward's checks of *p; LISA_ERR_NULL if schedule is NULL;
 * LISA_ERR_UNSUPPORTED if p->schedule is RESIDENT and that kernel does not
 * take the problem; LISA_ERR_HIP if no device is visible.  Host only;
 * enqueues nothing. */
lisa_status lisa_forward_schedule(const lisa_problem* p, int32_t* schedule);

/* The whole LiSA forward pass: Y = alpha G + (1 - alpha) L (see top).
 *   weights : [batch, heads, n, T] fp32 adaptive step weights w_k(i)
 *             [note §2.4 Eq. 10], or NULL for geometric weights of `beta`
 *             [note §2.2 Eq. 4].
 *   beta    : continuation probability in [0, 1); read only when weights is
 *             NULL.
 *   alpha   : [heads] fp32 mixing coefficients (device); not range-checked,
 *             values outside [0, 1] extrapolate.
 *   Y       : [batch, heads, n, d_v] output, dtype of the problem. */
lisa_status lisa_forward(const lisa_problem* p, const void* Q, const void* K, const void* V,
                         const float* weights, float beta, const float* alpha, void* Y,
                         void* workspace, size_t workspace_bytes, void* stream);

/* lisa_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments as for lisa_forward, without a workspace: the launch counters,
 * rank partials and statistics live in a fixed array of the library, 32 MiB
 * of device memory per GPU, which each GPU that runs this call holds until
 * the process ends.  The call allocates nothing (no hipMalloc, no library
 * routine that allocates) and, like lisa_forward, only enqueues work.
 *   - Limit: at most 8192 (batch, head) slices, and counters plus partials
 *     for the device's launch within 32 MiB (PVT-T stage 1, B = 32: 10 MB;
 *     one 200 x 320 sequence: 9 MB); a larger problem returns
 *     LISA_ERR_SCRATCH before anything is enqueued.
 *   - Every call on one GPU shares that GPU's array and finds the previous
 *     call's contents there; each completed call leaves the words that must
 *     start at zero (counters, tickets, the stall flag) at zero.  Calls that
 *     overlap on one GPU (other streams, other host threads) race and give
 *     undefined results: order them on one stream.
 *   - An abandoned wait (see Scheduling above) is not reported: with no
 *     workspace there is nothing for lisa_workspace_check to read, and the
 *     call clears the flag when it finishes.
 *   - Same kernels and results as lisa_forward for the same problem and
 *     inputs; the statistics are not left anywhere the other entry points
 *     (lisa_apply, lisa_backward_after_forward) can read. */
lisa_status lisa_forward_noalloc(const lisa_problem* p, const void* Q, const void* K, const void* V,
                                 const float* weights, float beta, const float* alpha, void* Y,
                                 void* stream);

/* lisa_forward that also records when each workgroup of the launch reached
 * each stage of the pass, for performance analysis [the stages of note §2.3
 * Eq. 8 / Algorithm 1: the statistics sweeps, their sums, the output].
 * Same arguments, work and Y as lisa_forward, plus
 *   stamps       : device array of stamps_count uint64_t (8-byte aligned);
 *                  workgroup w writes entry w * LISA_PHASES + k when it
 *                  reaches stage k (LISA_STAGE_*) of its first slice: the
 *                  device's constant 100 MHz clock (s_memrealtime); entry
 *                  w * LISA_PHASES + LISA_PHASES - 1 holds its group (high
 *                  32 bits) and its rank in the group (low).  A stage the
 *                  problem does not have leaves its entry as it was.
 *   stamps_count : at least (compute units) * LISA_PHASES, else LISA_ERR_PARAM.
 * Runs the resident kernel (LISA_SCHEDULE_RESIDENT) whatever p->schedule
 * asks, except STREAMING; only for problems it takes (bf16, ReLU features,
 * T <= 8, grids whose tiles fit a workgroup).  Others, and STREAMING, return
 * LISA_ERR_UNSUPPORTED before anything is enqueued. */
#define LISA_PHASES 16
enum {
  LISA_STAGE_START = 0,  /* rank taken */
  LISA_STAGE_STAGED,     /* K, V cells, weights, Q in LDS / registers */
  LISA_STAGE_KV,         /* partial of s and phi(K)^T V published */
  LISA_STAGE_LOCAL,      /* local branch and k = 0 term done */
  LISA_STAGE_S,          /* every rank's KV partial arrived; s formed */
  LISA_STAGE_M,          /* partial of M published */
  LISA_STAGE_MWAIT,      /* every rank's M partial arrived */
  LISA_STAGE_COMBINE,    /* this rank's share of the statistics written */
  LISA_STAGE_CWAIT,      /* every rank's share arrived */
  LISA_STAGE_FRAGS,      /* statistics fragments loaded */
  LISA_STAGE_OUT,        /* Y of every slice written */
  LISA_STAGE_END,        /* workgroup done */
  LISA_STAGE_KVSWEEP,    /* products of the KV sweep done, before publishing */
  LISA_STAGE_CSTAGED,    /* this rank's share of every partial loaded */
  LISA_STAGE_CSUMMED     /* that share summed, before it is written */
};
lisa_status lisa_forward_phases(const lisa_problem* p, const void* Q, const void* K, const void* V,
                                const float* weights, float beta, const float* alpha, void* Y,
                                void* workspace, size_t workspace_bytes, uint64_t* stamps,
                                size_t stamps_count, void* stream);

/* First stage alone: the d_h-space statistics of every (batch, head)
 * [note §2.3 Eq. 8]:
 *   s_out  [batch, heads, d_h]      s = sum_j phi(K_j)
 *   kv_out [batch, heads, d_h, d_v] phi(K)^T V
 *   m_out  [batch, heads, d_h, d_h] M = phi(K)^T Qt, Qt_i = phi(Q_i) / (phi(Q_i) . s + eps)
 * All three fp32, row-major; each may be NULL to skip that copy.  The
 * statistics are also left in the workspace, where lisa_apply reads them.
 * p->T is checked like everywhere else but all three are always formed. */
lisa_status lisa_reduce(const lisa_problem* p, const void* Q, const void* K, const void* V,
                        float* s_out, float* kv_out, float* m_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Second stage alone: the output pass of lisa_forward, using the statistics
 * that the last lisa_reduce on the same problem, inputs and workspace left
 * there.  lisa_reduce followed by lisa_apply computes the same Y as
 * lisa_forward, with the same kernels when T >= 3 (for T < 3 lisa_forward
 * skips the statistics it does not need).  Arguments as for lisa_forward. */
lisa_status lisa_apply(const lisa_problem* p, const void* Q, const void* K, const void* V,
                       const float* weights, float beta, const float* alpha, void* Y,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Walk-weight predictor [note §2.4, Eq. 10; supplementary Sec. 8]: the
 * adaptive weights of token i and head h are predicted from the token's
 * query and key concatenated, by a two-layer MLP and a softmax over the T
 * weights.  The note gives no widths, activation or biases; here
 *   w_i = softmax(W2 ReLU(W1 concat(Q_i, K_i) + b1) + b2),
 * per head, Q_i and K_i as given (before the feature map), query first.
 *   hidden : hidden width, a multiple of 32 in [32, 128]
 *   w1     : [heads, hidden, 2 d_h] fp32 (device)
 *   b1     : [heads, hidden] fp32
 *   w2     : [heads, T, hidden] fp32
 *   b2     : [heads, T] fp32
 * All four are 4-byte aligned device arrays owned by the caller. */
typedef struct lisa_weight_mlp {
  int32_t hidden;
  const float* w1;
  const float* b1;
  const float* w2;
  const float* b2;
} lisa_weight_mlp;

/* Workspace bytes for lisa_forward_mlp (the forward's workspace plus W1 in
 * the layout the kernel reads), or 0 if the problem or hidden is invalid
 * (T > 8 included). */
size_t lisa_forward_mlp_workspace_size(const lisa_problem* p, int32_t hidden);

/* The forward pass with the walk weights predicted inside the output pass
 * (no [batch, heads, n, T] weight tensor is read or written): the same Y as
 * lisa_forward given the predictor's weights.  With bf16 inputs the first
 * layer multiplies the exact bf16 inputs by W1 rounded to bf16 (as the walk
 * rounds its P_k), with fp32 sums; everything else is fp32.  mlp NULL or a NULL array:
 * LISA_ERR_NULL; hidden out of range or T > 8: LISA_ERR_PARAM; other arguments and
 * errors as for lisa_forward with weights == NULL, the workspace
 * lisa_forward_mlp_workspace_size bytes. */
lisa_status lisa_forward_mlp(const lisa_problem* p, const void* Q, const void* K, const void* V,
                             const lisa_weight_mlp* mlp, const float* alpha, void* Y,
                             void* workspace, size_t workspace_bytes, void* stream);

/* A LiSA attention layer around the operator [note §2.1: n tokens X are
 * projected to Q, K, V; the operator replaces the attention of DeiT-T and
 * PVT-T]: [Q | K | V] = X Wqkv^T + bqkv, head h taking channels
 * 64 h .. 64 h + 63, O = lisa_forward(Q, K, V) per head, and
 * Y = concat_h(O_h) Wo^T + bo.  C = heads * 64 (p->d_h = p->d_v = 64).
 *   X     : [batch, n, C], dtype of the problem (device)
 *   w_qkv : [3 C, C] (the torch Linear layout: out x in), dtype of the problem
 *   b_qkv : [3 C] fp32
 *   w_o   : [C, C], dtype of the problem;  b_o : [C] fp32
 *   weights, beta, alpha : as for lisa_forward
 *   Y     : [batch, n, C], dtype of the problem; X and Y must not overlap
 *           each other or the workspace (LISA_ERR_PARAM)
 * Q, K, V and O live in the workspace (lisa_attention_workspace_size bytes,
 * 256-byte aligned, zero-filled before its first use), in the problem's
 * dtype: with bf16 inputs each is rounded once, as between separate layers.
 * With one head in bf16 (where lisa_forward takes the resident kernel) the
 * output projection is applied in the operator's output stage instead: O is
 * rounded to bf16 as the product's operand, the same values as stored.
 * The projections run on MFMA with fp32 sums.  Errors as for lisa_forward;
 * X, Y and the weights need 16-byte alignment, the biases 4. */
size_t lisa_attention_workspace_size(const lisa_problem* p);
lisa_status lisa_attention_forward(const lisa_problem* p, const void* X, const void* w_qkv,
                                   const float* b_qkv, const void* w_o, const float* b_o,
                                   const float* weights, float beta, const float* alpha, void* Y,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass: the gradients of lisa_forward's Y, contracted with the
 * output gradient dY, for every input.  The note trains every model it
 * reports [note §3] and gives no backward formulas; these are the exact
 * derivatives of the forward pass [note §2.1-§2.4] (the ReLU's derivative at
 * 0 is taken as 0).  The call recomputes the slice statistics (as
 * lisa_reduce) and then runs the token passes; all arithmetic is fp32.
 *   Q, K, V, weights, beta, alpha : as for lisa_forward (device)
 *   dY       : [batch, heads, n, d_v] output gradient, dtype of the problem
 *   dQ, dK, dV : [batch, heads, n, d] gradients, dtype of the problem
 *                (bf16: rounded once, to nearest even)
 *   dweights : [batch, heads, n, T] fp32 gradient of the adaptive weights;
 *              may be NULL to skip it; ignored with geometric weights (no
 *              gradient for beta is formed)
 *   dalpha   : [heads] fp32 gradient of alpha (summed over the batch)
 * Outputs must not overlap any input, each other or the workspace
 * (LISA_ERR_PARAM), as is T > 8.  Workspace: lisa_backward_workspace_size
 * bytes (0 for an invalid problem or T > 8), 256-byte
 * aligned, zero-filled before its first use like lisa_forward's; it also
 * serves lisa_forward, lisa_reduce and lisa_apply of the same problem. */
size_t lisa_backward_workspace_size(const lisa_problem* p);
lisa_status lisa_backward(const lisa_problem* p, const void* Q, const void* K, const void* V,
                          const float* weights, float beta, const float* alpha, const void* dY,
                          void* dQ, void* dK, void* dV, float* dweights, float* dalpha,
                          void* workspace, size_t workspace_bytes, void* stream);

/* The gradients of lisa_backward, for a training step whose forward pass
 * (lisa_forward, lisa_forward_mlp or lisa_reduce) ran just before on the
 * same problem and the same Q, K, V, with this workspace, on this stream:
 * with T >= 3 the slice statistics s, phi(K)^T V and M that call left in the
 * workspace are used as they are and the statistics launch is skipped (with
 * T < 3 the forward forms no M, and they are recomputed as lisa_backward
 * does).  The results equal lisa_backward's bit for bit.  No other call may
 * use the workspace in between: the library cannot check this, and
 * statistics of other inputs give wrong gradients without an error.
 * Arguments, errors and workspace as for lisa_backward. */
lisa_status lisa_backward_after_forward(const lisa_problem* p, const void* Q, const void* K, const void* V,
                                        const float* weights, float beta, const float* alpha,
                                        const void* dY, void* dQ, void* dK, void* dV, float* dweights,
                                        float* dalpha, void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Whether a call on `workspace` abandoned a wait (see Scheduling above).
 * Unlike the other entry points this call synchronises: it waits for the
 * work enqueued on `stream` so far, reads the workspace's stall flag, clears
 * it, and returns LISA_ERR_STALLED if it was set (the outputs of the calls on
 * this workspace since the previous check are then undefined; the workspace
 * itself is ready for further calls), else LISA_OK.  The flag is word 1 of
 * the launch counters at the start of every workspace, whose place no
 * problem moves.  Errors: NULL workspace (LISA_ERR_NULL), fewer than 256
 * bytes or not 256-byte aligned (LISA_ERR_WORKSPACE), a failed HIP call
 * (LISA_ERR_HIP). */
lisa_status lisa_workspace_check(void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* lisa_status_str(lisa_status s);

#ifdef __cplusplus
}
#endif

#endif /* LISA_H */
