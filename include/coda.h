/*
 * coda.h - C ABI of the fused GEMM -> residual -> RMSNorm -> GEMM chain for
 * AMD MI355X (gfx950), forward and backward.
 *
 * The operation (CODA: Rewriting Transformer Blocks as GEMM-Epilogue Programs,
 * hotdry blog page, section "GEMM-Residual-RMSNorm-GEMM 重参数化"):
 *
 *     y = RMSNorm(x @ W0 + z, gamma) @ W1
 *
 * evaluated in the reparameterised order of the same section, where the row
 * scale r commutes with the second GEMM:
 *
 *     h = x @ W0 + z,   g = h * gamma,   r_i = 1 / sqrt(mean_j h_ij^2 + eps),
 *     y = r (row-broadcast) * (g @ W1).
 *
 * The first GEMM's epilogue adds the residual, stores h and g and emits tile
 * partial sums of squares; a light reduction turns them into r; the second
 * GEMM's epilogue applies r (same section, steps 1-3).
 *
 * Backward of L = <dY, y> (same page, section "反向传播的 GEMM-Epilogue 结构":
 * the backward keeps the GEMM-epilogue form and the row statistic s is taken at
 * the GEMM boundary as s = sum_cols(dY * y)):
 *
 *     s_i   = sum_n dY_in y_in
 *     G     = dY @ W1^T               (epilogue: da and dgamma column partials)
 *     da_ij = r_i gamma_j G_ij - s_i r_i^2 h_ij / D
 *     dgamma_j = sum_i G_ij r_i h_ij
 *     dW1   = (r * g)^T @ dY          (r * g rounded once to bf16 before the GEMM)
 *
 * Conventions for every entry point:
 *   - All tensors are dense and row-major. bf16 means IEEE bfloat16 (stored as
 *     uint16); f32 means IEEE binary32. W0 is [K0, D] and W1 is [D, N] ([in, out]).
 *   - Pointers are device pointers (HIP device memory), 16-byte aligned. The
 *     caller owns every buffer, including the workspace; the library never
 *     allocates, frees or synchronises. Work is enqueued on `stream` (a
 *     hipStream_t; NULL is the default stream) and the call returns at once.
 *     Calls on one stream with distinct outputs/workspaces are independent; the
 *     library keeps no global state.
 *   - Shapes: 1 <= M <= 2^22 (any value; the last row tile is masked); K0, D
 *     and N are multiples of 64 in [64, 2^20] (a last column tile narrower than
 *     256 is masked per 64 columns); and every GEMM of the call has
 *     at most 2^23 output tiles of 256 x 256 (its launch stays within 2^32
 *     work-items). Anything else returns CODA_ERR_SHAPE.
 *   - eps must be finite and > 0.
 *   - Arguments are validated on the host before anything is launched; on any
 *     error nothing is enqueued and the status is returned. A failed launch
 *     returns CODA_ERR_HIP. Device faults surface at the caller's next sync.
 *   - NaN/Inf inputs are not trapped; they propagate row-locally (a non-finite
 *     value in row i of x/z/dY/h/y affects row i's outputs and, through the
 *     column sums, dgamma/dW1).
 */
#ifndef CODA_H
#define CODA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum below also names the smallest and largest int32 (the *_RANGE_MIN_ / *_RANGE_MAX_
 * sentinels, which no function accepts): that fixes each enum's range to all of int32, so any int a C
 * caller passes (e.g. through ctypes) is a defined value of the type, and the validators reject it
 * with CODA_ERR_ARG instead of the C++ implementation reading an out-of-range enum. */
#define CODA_ENUM_MIN_ (-0x7fffffff - 1)
#define CODA_ENUM_MAX_ 0x7fffffff

typedef enum {
  CODA_OK = 0,
  CODA_ERR_NULL = 1,      /* a required pointer is NULL                      */
  CODA_ERR_SHAPE = 2,     /* unsupported or inconsistent sizes               */
  CODA_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned                */
  CODA_ERR_WORKSPACE = 4, /* workspace NULL or smaller than required          */
  CODA_ERR_ARG = 5,       /* bad scalar argument (eps, dtype, op, layout)     */
  CODA_ERR_HIP = 6,       /* a HIP launch failed                              */
  CODA_STATUS_RANGE_MIN_ = CODA_ENUM_MIN_, CODA_STATUS_RANGE_MAX_ = CODA_ENUM_MAX_
} coda_status_t;

typedef enum {
  CODA_BF16 = 0,
  CODA_F32 = 1,
  CODA_DTYPE_RANGE_MIN_ = CODA_ENUM_MIN_, CODA_DTYPE_RANGE_MAX_ = CODA_ENUM_MAX_
} coda_dtype_t;

/* Operations, for coda_workspace_bytes. */
typedef enum {
  CODA_OP_FWD = 0,          /* coda_fwd                      */
  CODA_OP_BWD = 1,          /* coda_bwd                      */
  CODA_OP_UNFUSED_FWD = 2,  /* coda_unfused_ref(CODA_OP_FWD)  */
  CODA_OP_UNFUSED_BWD = 3,  /* coda_unfused_ref(CODA_OP_BWD)  */
  CODA_OP_FWD_SWIGLU = 4,   /* coda_fwd_swiglu */
  CODA_OP_BWD_SWIGLU = 5,   /* coda_bwd_swiglu */
  CODA_OP_CE_FWD = 6,       /* coda_ce_fwd (pass the vocabulary size V as N) */
  CODA_OP_CE_BWD = 7,       /* coda_ce_bwd (none) */
  CODA_OP_UNFUSED_FWD_SWIGLU = 8, /* coda_unfused_ref(CODA_OP_FWD_SWIGLU) */
  CODA_OP_UNFUSED_BWD_SWIGLU = 9, /* coda_unfused_ref(CODA_OP_BWD_SWIGLU) */
  CODA_OP_UNFUSED_CE_FWD = 10,    /* coda_unfused_ref(CODA_OP_CE_FWD) (V as N) */
  CODA_OP_UNFUSED_CE_BWD = 11,    /* coda_unfused_ref(CODA_OP_CE_BWD) (V as N) */
  CODA_OP_RANGE_MIN_ = CODA_ENUM_MIN_, CODA_OP_RANGE_MAX_ = CODA_ENUM_MAX_
} coda_op_t;

/* Forward arguments.
 *   in : x [M,K0] bf16, W0 [K0,D] bf16, z [M,D] bf16 (residual), gamma [D] bf16,
 *        W1 [D,N] bf16 (columns 2f / 2f+1 are the gate / up pair of feature f;
 *        the chain's arithmetic does not depend on this labelling).
 *   out: h [M,D] bf16 (= x@W0 + z, rounded once from fp32),
 *        g [M,D] bf16 (= h*gamma rounded once from the fp32 h),
 *        r [M] f32 (row inverse RMS), y [M,N] in y_dtype.
 * h, g, r and y are what the backward needs; the fused forward writes all four. */
typedef struct {
  int64_t M, K0, D, N;
  float eps;
  const void* x;
  const void* W0;
  const void* z;
  const void* gamma;
  const void* W1;
  void* h;
  void* g;
  float* r;
  void* y;
  coda_dtype_t y_dtype;
} coda_fwd_args_t;

/* Backward arguments.
 *   in : dY [M,N] bf16; the forward's saved y [M,N] bf16, h [M,D] bf16,
 *        g [M,D] bf16, r [M] f32; gamma [D] bf16; W1 [D,N] bf16.
 *   out: da [M,D] in da_dtype (gradient w.r.t. the RMSNorm input h),
 *        dgamma [D] f32, dW1 [D,N] in dW1_dtype, s [M] f32 (the row statistic). */
typedef struct {
  int64_t M, D, N;
  const void* dY;
  const void* y;
  const void* h;
  const void* g;
  const float* r;
  const void* gamma;
  const void* W1;
  void* da;
  float* dgamma;
  void* dW1;
  float* s;
  coda_dtype_t da_dtype;
  coda_dtype_t dW1_dtype;
} coda_bwd_args_t;

/* Backward through the chain's first GEMM and its residual, h = x @ W0 + z
 * (hotdry blog, section "GEMM-Residual-RMSNorm-GEMM 重参数化", for the
 * forward; kucoin page, section "実験結果", which evaluates the backward of the
 * whole GEMM-Residual-RMSNorm-GEMM chain), for an upstream gradient dh of h
 * (coda_bwd's da stored as bf16, plus whatever gradient the residual stream
 * adds, which this chain does not model):
 *     dz = dh            (nothing to compute: the caller uses dh itself)
 *     dx = dh @ W0^T     dW0 = x^T @ dh
 *   in : dh [M,D] bf16, x [M,K0] bf16, W0 [K0,D] bf16.
 *   out: dx [M,K0] in dx_dtype, dW0 [K0,D] in dW0_dtype.
 * Two launches of the shared mainloop with store-only epilogues; no workspace.
 * Shapes as for coda_fwd (K0 and D multiples of 64, any M >= 1). */
typedef struct {
  int64_t M, K0, D;
  const void* dh;
  const void* x;
  const void* W0;
  void* dx;
  void* dW0;
  coda_dtype_t dx_dtype;
  coda_dtype_t dW0_dtype;
} coda_bwd_gemm0_args_t;

/* SwiGLU on the chain's output (hotdry blog, section "成对激活的寄存器级融合":
 * paired features sit in adjacent output columns, so the gated activation is
 * applied in the epilogue that produces the pair). Column 2f of y is gate f and
 * column 2f+1 is up f; F = N/2 features:
 *     o_if = silu(y_i,2f) * y_i,2f+1,   silu(v) = v / (1 + exp(-v)).
 * The forward is coda_fwd with GEMM1's epilogue also emitting o (from the fp32
 * y; y itself is still stored, in bf16 as the backward takes it: chain.y_dtype
 * must be CODA_BF16). N must be a multiple of 128. Workspace: as coda_fwd
 * (coda_workspace_bytes(CODA_OP_FWD_SWIGLU, ...)). */
typedef struct {
  coda_fwd_args_t chain; /* as for coda_fwd */
  void* o;               /* out: [M, N/2] in o_dtype */
  coda_dtype_t o_dtype;
} coda_fwd_swiglu_args_t;

/* Backward of the SwiGLU block for an output projection out = o @ W2 and
 * L = <dOut, out> (same page, sections on pairwise activations — their backward
 * is a dimension-expanding epilogue — and on the backward's GEMM-epilogue form,
 * where the row statistic s is accumulated by the GEMM epilogue that produces
 * the gradient of y):
 *     dO  = dOut @ W2^T, its epilogue expanding each feature to its pair:
 *           dY_i,2f = dO_if y_i,2f+1 silu'(y_i,2f),  dY_i,2f+1 = dO_if silu(y_i,2f)
 *           and the partial sums of s_i = sum_n dY_in y_in (fp32 dY, saved bf16 y);
 *     then the chain's backward on this dY: da, dgamma, dW1 (as coda_bwd), and
 *     dW2 = o^T @ dOut.
 *   in : dOut [M,E] bf16; W2 [F,E] bf16 (F = N/2); the forward's saved
 *        o [M,F] bf16, y [M,N] bf16, h [M,D] bf16, g [M,D] bf16, r [M] f32;
 *        gamma [D] bf16; W1 [D,N] bf16.
 *   out: dY [M,N] bf16, da [M,D] in da_dtype, dgamma [D] f32, dW1 [D,N] in
 *        dW1_dtype, dW2 [F,E] in dW2_dtype, s [M] f32.
 * N a multiple of 128, E a multiple of 64 in [64, 2^20]. */
typedef struct {
  int64_t M, D, N, E;
  const void* dOut;
  const void* W2;
  const void* o;
  const void* y;
  const void* h;
  const void* g;
  const float* r;
  const void* gamma;
  const void* W1;
  void* dY;
  void* da;
  float* dgamma;
  void* dW1;
  void* dW2;
  float* s;
  coda_dtype_t da_dtype;
  coda_dtype_t dW1_dtype;
  coda_dtype_t dW2_dtype;
} coda_bwd_swiglu_args_t;

/* Cross-entropy on an LM-head GEMM (hotdry blog, section "五类 Epilogue 原语": the
 * stateful-transform primitive keeps tile-level online log-sum-exp and cross-entropy
 * statistics; kucoin, section "五つの「ブロック」": block log-sum-exp, running max and
 * sum-exp). For hidden states h [M, D], an output weight W [V, D] (one row per
 * vocabulary entry, the nn.Linear / tied-embedding layout) and targets t [M]:
 *     logits = h @ W^T (not stored unless asked for, see below),
 *     lse_i  = log sum_v exp(logits_iv),   loss_i = lse_i - logits_i,t_i.
 * The logits GEMM's epilogue reduces each (row, 64-column) tile to its max m and
 * sum exp(logit - m) and picks out the target logit; a row kernel combines the
 * tile statistics in a fixed order. A target outside [0, V) marks an ignored row:
 * its loss is 0 (lse is still written). D and V multiples of 64 in [64, 2^20]
 * (Llama-3's V = 128256 = 501 * 256).
 *   in : h [M,D] bf16, W [V,D] bf16, targets [M] int64.
 *   out: lse [M] f32, loss [M] f32 (per row; a mean is the caller's sum / count);
 *        logits [M,V] f32, optional (NULL: not stored): the same epilogue also stores the
 *        fp32 logits, which coda_ce_bwd then reads instead of recomputing them -- 4 M V
 *        bytes (4.2 GB at M = 8192, V = 128256) traded for the backward's logits GEMM.
 * Workspace: coda_workspace_bytes(CODA_OP_CE_FWD, M, D, V). */
typedef struct {
  int64_t M, D, V;
  const void* h;
  const void* W;
  const int64_t* targets;
  float* lse;
  float* loss;
  float* logits;
} coda_ce_fwd_args_t;

/* Backward of L = sum_i dloss_i loss_i for the forward's lse (same sections; the
 * backward of a tile-local epilogue is again tile-local, on the logits recomputed by
 * the same GEMM):
 *     dlogits_iv = dloss_i (exp(logits_iv - lse_i) - [v = t_i]), 0 on ignored rows,
 *     dh = dlogits @ W,   dW = dlogits^T @ h.
 *   in : h, W, targets as in the forward; lse [M] f32 (the forward's); dloss [M] f32;
 *        logits [M,V] f32, optional: the forward's stored logits (NULL: recomputed by the
 *        GEMM). Given, a row kernel reads them for dlogits (the same values: the stored
 *        logits are the recomputing GEMM's accumulators).
 *   out: dlogits [M,V] bf16 (the operand of the two products, written as an output),
 *        dh [M,D] in dh_dtype, dW [V,D] in dW_dtype. No workspace. */
typedef struct {
  int64_t M, D, V;
  const void* h;
  const void* W;
  const int64_t* targets;
  const float* lse;
  const float* dloss;
  void* dlogits;
  void* dh;
  void* dW;
  coda_dtype_t dh_dtype;
  coda_dtype_t dW_dtype;
  const float* logits;
} coda_ce_bwd_args_t;

/* Operand layouts for coda_gemm. */
typedef enum {
  CODA_ROW = 0, /* A: element (m,k) at A[m*lda + k];  B: element (k,n) at B[k*ldb + n] */
  CODA_COL = 1, /* A: element (m,k) at A[k*lda + m];  B: element (k,n) at B[n*ldb + k] */
  CODA_LAYOUT_RANGE_MIN_ = CODA_ENUM_MIN_, CODA_LAYOUT_RANGE_MAX_ = CODA_ENUM_MAX_
} coda_layout_t;

/* Plain GEMM C[M,N] = A[M,K] @ B[K,N] with bf16 operands and fp32 accumulation,
 * output in c_dtype with leading dimension ldc. This is the mainloop every
 * fused kernel shares, with a store-only epilogue; the unfused baseline is
 * built from it. M >= 1, N and K multiples of 64, lda/ldb/ldc >= the
 * contiguous extent and multiples of 8. */
typedef struct {
  int64_t M, N, K;
  const void* A;
  int64_t lda;
  coda_layout_t a_layout;
  const void* B;
  int64_t ldb;
  coda_layout_t b_layout;
  void* C;
  int64_t ldc;
  coda_dtype_t c_dtype;
} coda_gemm_args_t;

/* Bytes of device workspace `op` needs for these sizes (0 when none). The
 * workspace of the fused forward holds the partial sums of squares; the
 * fused backward holds bf16(r*g) transposed, [D, M rounded up to 64], and the dgamma column partials (the
 * SwiGLU backward also the partial sums of s); the unfused baseline also holds
 * its materialised intermediates. When the backward's data-gradient GEMM has
 * fewer than 192 tiles of 256 x 256 (tiles = ceil(M/256) * ceil(D/256); few rows M, e.g. a
 * data-parallel shard),
 * its contraction over N is split into S = min(ceil(256 / tiles), 8, N / 256)
 * slices and the workspace also holds their fp32 partial products [S, M, D]
 * (the dgamma partials then have ceil(M / 8) rows instead of ceil(M / 128)).
 * The forward splits GEMM0 by the same rule (tiles = ceil(M/256) * ceil(D/256)); its
 * workspace, sized without K0, then also holds min(ceil(256 / tiles), 8) fp32
 * partial products [., M, D]. */
size_t coda_workspace_bytes(coda_op_t op, int64_t M, int64_t D, int64_t N);

/* Host-only argument checks (no HIP call). Return CODA_OK or the first error. */
coda_status_t coda_validate_fwd(const coda_fwd_args_t* a, const void* ws, size_t ws_bytes);
coda_status_t coda_validate_bwd(const coda_bwd_args_t* a, const void* ws, size_t ws_bytes);
coda_status_t coda_validate_gemm(const coda_gemm_args_t* a);
coda_status_t coda_validate_bwd_gemm0(const coda_bwd_gemm0_args_t* a);
coda_status_t coda_validate_fwd_swiglu(const coda_fwd_swiglu_args_t* a, const void* ws, size_t ws_bytes);
coda_status_t coda_validate_bwd_swiglu(const coda_bwd_swiglu_args_t* a, const void* ws, size_t ws_bytes);
coda_status_t coda_validate_ce_fwd(const coda_ce_fwd_args_t* a, const void* ws, size_t ws_bytes);
coda_status_t coda_validate_ce_bwd(const coda_ce_bwd_args_t* a);
/* Checks of coda_unfused_ref's arguments (op = CODA_OP_FWD, CODA_OP_BWD, CODA_OP_FWD_SWIGLU,
 * CODA_OP_BWD_SWIGLU, CODA_OP_CE_FWD or CODA_OP_CE_BWD). */
coda_status_t coda_validate_unfused(coda_op_t op, const void* args, const void* ws, size_t ws_bytes);

/* Fused forward: GEMM0 + epilogue (residual, h, g, one sum-of-squares partial per row and
 * 256-column tile, its four waves' sums added in the block) -> row-statistic combine (r) ->
 * GEMM1 + epilogue (row scale r). The combine is the light auxiliary reduction between the two
 * epilogues (hotdry blog, section "GEMM-Residual-RMSNorm-GEMM 重参数化", step 2); GEMM1's epilogue does it
 * itself, with no kernel of its own, when ceil(D / 256) <= 32 and GEMM1 has at most 512 tiles of
 * 256 x 256 (ceil(M / 256) * ceil(N / 256)): every tile repeats it, which costs more than a
 * separate launch once GEMM1 runs more than two waves of tiles. */
coda_status_t coda_fwd(const coda_fwd_args_t* a, void* ws, size_t ws_bytes, void* stream);

/* The fused forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same kernels as coda_fwd, with the
 * sum-of-squares partials kept in a device array of the library's own, CODA_NOALLOC_SCRATCH_BYTES
 * (16 MiB), which every GPU the library runs on holds until the process ends; no workspace argument,
 * and no allocation or free of any kind. GEMM0 is never split over its contraction here (coda_fwd
 * splits it when its tiles cannot fill the chip), so the partials need only M * ceil(D / 256) * 4 bytes.
 *   - Returns CODA_ERR_WORKSPACE, launching nothing, when M * ceil(D / 256) * 4 exceeds the 16 MiB
 *     (e.g. M > 262144 rows at D = 4096); every other check and status is coda_fwd's.
 *   - All calls on one GPU share that GPU's array: calls that may overlap on one GPU (on different
 *     streams, or from several threads) race and must be ordered by the caller. A call needs nothing
 *     from the previous one (its partials are written in full before they are read).
 *   - The first call on a device looks the array's device address up (hipGetSymbolAddress with
 *     that device current) and keeps it; a failed lookup returns CODA_ERR_HIP. */
#define CODA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
coda_status_t coda_validate_fwd_noalloc(const coda_fwd_args_t* a);
coda_status_t coda_fwd_noalloc(const coda_fwd_args_t* a, void* stream);

/* Fused backward: bf16(r*g) transposed (so the dW1 GEMM's left operand is
 * contiguous along its contraction) -> dW1 = bf16(r*g)^T @ dY, which also takes
 * the row statistic s_i = sum_n dY_in y_in from the dY tiles it already streams
 * (partials of 128 columns, hotdry blog, section "反向传播的 GEMM-Epilogue 结构":
 * s in the kernel that reads dY) -> s, their fixed-order sum -> G = dY@W1^T with the
 * RMSNorm-backward epilogue (da, dgamma column partials) -> dgamma, the partials'
 * fixed-order sum. With D <= 3840 (fewer than 16 of the dW1 GEMM's 256-row tiles,
 * too few to deal a K step's 64 rows over) a row kernel over dY and y computes s
 * instead. */
coda_status_t coda_bwd(const coda_bwd_args_t* a, void* ws, size_t ws_bytes, void* stream);

/* The stages of coda_fwd and coda_bwd, one kernel each (two for a split GEMM), for callers that
 * interleave their own work or time the kernels. Running stages 0..n-1 in order
 * on one stream is exactly coda_fwd / coda_bwd; a stage reads what earlier
 * stages wrote into the outputs and the workspace. (A stage whose GEMM is split
 * over its contraction -- see coda_workspace_bytes -- launches the GEMM and a row
 * kernel that finishes its epilogue.) Each call validates the
 * whole argument set; a stage index out of range returns CODA_ERR_ARG.
 *   forward : 0 GEMM0 + residual/h/g/sum-of-squares epilogue, 1 r combine (launches
 *             nothing where GEMM1's epilogue combines r itself, see coda_fwd),
 *             2 GEMM1 + row-scale epilogue
 *   backward: 0 bf16(r*g) transposed for the dW1 GEMM, 1 dW1 GEMM (and s's
 *             partials, D > 3840), 2 s (the partials' sum, or the row kernel),
 *             3 G = dY@W1^T + RMSNorm-backward epilogue, 4 dgamma (the column
 *             partials' sum) */
#define CODA_FWD_STAGES 3
#define CODA_BWD_STAGES 5
coda_status_t coda_fwd_stage(int stage, const coda_fwd_args_t* a, void* ws, size_t ws_bytes, void* stream);
coda_status_t coda_bwd_stage(int stage, const coda_bwd_args_t* a, void* ws, size_t ws_bytes, void* stream);

/* Unfused baseline with the same mainloop and separate row kernels: the conventional chain the
 * fusion is measured against, three operators in series with the intermediate written to device
 * memory and read back between them (kucoin page, section "CODA：「尾声」に隠された宝物").
 *   op = CODA_OP_FWD, args = coda_fwd_args_t*: t = x@W0 (bf16, workspace) ->
 *     add+RMSNorm row kernel (h, r, n = bf16(r*h*gamma) into the workspace) ->
 *     y = n@W1. Writes h, r and y; g is not written (this chain feeds n, not g,
 *     to the second GEMM).
 *   op = CODA_OP_BWD, args = coda_bwd_args_t*: a row kernel for s and bf16(r*g)
 *     (row layout) -> G = dY@W1^T stored as bf16 in the workspace ->
 *     RMSNorm-backward row kernel (da, dgamma partials) -> dgamma combine ->
 *     dW1 GEMM on the row-layout bf16(r*g).
 *   op = CODA_OP_FWD_SWIGLU, args = coda_fwd_swiglu_args_t*: the fused chain
 *     forward (coda_fwd, y stored bf16) -> a row kernel o = silu(gate) * up from
 *     the stored y. Only the SwiGLU step is unfused.
 *   op = CODA_OP_BWD_SWIGLU, args = coda_bwd_swiglu_args_t*: dO = dOut@W2^T
 *     stored as bf16 in the workspace -> a row kernel (dY from dO and the saved
 *     y, s from the fp32 dY, bf16(r*g)) -> the fused chain backward's dgrad and
 *     dW1 GEMMs -> dW2. Only the SwiGLU step is unfused.
 *   op = CODA_OP_CE_FWD, args = coda_ce_fwd_args_t*: the logits h@W^T stored as
 *     fp32 in the workspace ([M, V]) -> a row kernel for lse and loss.
 *   op = CODA_OP_CE_BWD, args = coda_ce_bwd_args_t*: the logits stored as fp32
 *     in the workspace -> a row kernel for dlogits -> the same dh and dW GEMMs.
 *   (Both ignore the structs' optional logits pointer.) */
coda_status_t coda_unfused_ref(coda_op_t op, const void* args, void* ws, size_t ws_bytes, void* stream);

/* SwiGLU forward and backward (see coda_fwd_swiglu_args_t, coda_bwd_swiglu_args_t). */
coda_status_t coda_fwd_swiglu(const coda_fwd_swiglu_args_t* a, void* ws, size_t ws_bytes, void* stream);
coda_status_t coda_bwd_swiglu(const coda_bwd_swiglu_args_t* a, void* ws, size_t ws_bytes, void* stream);

/* Cross-entropy forward and backward (see coda_ce_fwd_args_t, coda_ce_bwd_args_t). */
coda_status_t coda_ce_fwd(const coda_ce_fwd_args_t* a, void* ws, size_t ws_bytes, void* stream);
coda_status_t coda_ce_bwd(const coda_ce_bwd_args_t* a, void* stream);

/* Backward through the first GEMM (see coda_bwd_gemm0_args_t): dx, then dW0. */
coda_status_t coda_bwd_gemm0(const coda_bwd_gemm0_args_t* a, void* stream);

/* Plain GEMM (see coda_gemm_args_t); needs no workspace. */
coda_status_t coda_gemm(const coda_gemm_args_t* a, void* stream);

/* Static description of a status code. */
const char* coda_status_string(coda_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* CODA_H */
