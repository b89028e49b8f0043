// Host-only part of the C ABI: workspace sizes, argument validation and status
// strings. Nothing here calls HIP, so the checks run (and are tested) without a GPU.
#include <math.h>

#include "coda.h"
#include "coda_internal.h"

using namespace coda;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dim_ok(int64_t v) { return v >= kDimQuantum && v <= kMaxDim && v % kDimQuantum == 0; }

bool rows_ok(int64_t M) { return M >= 1 && M <= kMaxRows; }

// A GEMM's grid (one 512-thread block per 256 x 256 output tile) fits a launch: at most 2^32 - 1 work-items.
bool grid_ok(int64_t rows, int64_t cols) { return ceil_div(rows, kBM) * ceil_div(cols, kBN) * kThreads <= 0xFFFFFFFFll; }

bool dtype_ok(coda_dtype_t t) { return t == CODA_BF16 || t == CODA_F32; }

// First failing pointer check over a list: NULL beats misalignment.
coda_status_t check_ptrs(const void* const* ps, int n) {
  for (int i = 0; i < n; ++i)
    if (ps[i] == nullptr) return CODA_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (!aligned16(ps[i])) return CODA_ERR_ALIGN;
  return CODA_OK;
}

coda_status_t check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return CODA_OK;
  if (ws == nullptr || ws_bytes < need) return CODA_ERR_WORKSPACE;
  if (!aligned16(ws)) return CODA_ERR_ALIGN;
  return CODA_OK;
}


size_t unfused_fwd_ws(int64_t M, int64_t D) { return 2 * align256(size_t(M) * size_t(D) * 2); }

size_t unfused_bwd_ws(int64_t M, int64_t D) {
  return 2 * align256(size_t(M) * size_t(D) * 2) +
         align256(size_t(ceil_div(M, kUnfusedBwdRows)) * size_t(D) * 4);
}

coda_status_t validate_fwd_common(const coda_fwd_args_t* a, bool need_g) {
  if (a == nullptr) return CODA_ERR_NULL;
  const void* ps[] = {a->x, a->W0, a->z, a->gamma, a->W1, a->h, a->r, a->y, a->g};
  coda_status_t st = check_ptrs(ps, need_g ? 9 : 8);
  if (st != CODA_OK) return st;
  if (!need_g && a->g != nullptr && !aligned16(a->g)) return CODA_ERR_ALIGN;
  if (!rows_ok(a->M) || !dim_ok(a->K0) || !dim_ok(a->D) || !dim_ok(a->N)) return CODA_ERR_SHAPE;
  if (!grid_ok(a->M, a->D) || !grid_ok(a->M, a->N)) return CODA_ERR_SHAPE;
  if (!(isfinite(a->eps) && a->eps > 0.0f)) return CODA_ERR_ARG;
  if (!dtype_ok(a->y_dtype)) return CODA_ERR_ARG;
  return CODA_OK;
}

coda_status_t validate_bwd_common(const coda_bwd_args_t* a) {
  if (a == nullptr) return CODA_ERR_NULL;
  const void* ps[] = {a->dY, a->y, a->h, a->g, a->r, a->gamma, a->W1, a->da, a->dgamma, a->dW1, a->s};
  coda_status_t st = check_ptrs(ps, 11);
  if (st != CODA_OK) return st;
  if (!rows_ok(a->M) || !dim_ok(a->D) || !dim_ok(a->N)) return CODA_ERR_SHAPE;
  if (!grid_ok(a->M, a->D) || !grid_ok(a->D, a->N)) return CODA_ERR_SHAPE;
  if (!dtype_ok(a->da_dtype) || !dtype_ok(a->dW1_dtype)) return CODA_ERR_ARG;
  return CODA_OK;
}

coda_status_t validate_ce_fwd_common(const coda_ce_fwd_args_t* a) {
  if (a == nullptr) return CODA_ERR_NULL;
  const void* ps[] = {a->h, a->W, a->targets, a->lse, a->loss};
  coda_status_t st = check_ptrs(ps, 5);
  if (st != CODA_OK) return st;
  if (!rows_ok(a->M) || !dim_ok(a->D) || !dim_ok(a->V) || !grid_ok(a->M, a->V)) return CODA_ERR_SHAPE;
  if (a->logits != nullptr && !aligned16(a->logits)) return CODA_ERR_ALIGN;  // optional output
  return CODA_OK;
}

coda_status_t validate_bwd_swiglu_common(const coda_bwd_swiglu_args_t* a) {
  if (a == nullptr) return CODA_ERR_NULL;
  const void* ps[] = {a->dOut, a->W2, a->o, a->y, a->h, a->g, a->r, a->gamma, a->W1, a->dY, a->da, a->dgamma,
                      a->dW1, a->dW2, a->s};
  coda_status_t st = check_ptrs(ps, 15);
  if (st != CODA_OK) return st;
  if (!rows_ok(a->M) || !dim_ok(a->D) || !dim_ok(a->N) || !dim_ok(a->E) || a->N % 128) return CODA_ERR_SHAPE;
  if (!grid_ok(a->M, a->D) || !grid_ok(a->D, a->N) || !grid_ok(a->M, a->N / 2) || !grid_ok(a->N / 2, a->E))
    return CODA_ERR_SHAPE;
  if (!dtype_ok(a->da_dtype) || !dtype_ok(a->dW1_dtype) || !dtype_ok(a->dW2_dtype)) return CODA_ERR_ARG;
  return CODA_OK;
}

}  // namespace

extern "C" {

size_t coda_workspace_bytes(coda_op_t op, int64_t M, int64_t D, int64_t N) {
  if (!rows_ok(M) || !dim_ok(D)) return 0;
  switch (op) {
    case CODA_OP_FWD: return fwd_ws(M, D);
    case CODA_OP_BWD: return dim_ok(N) ? bwd_chain_ws(M, D, N) : 0;
    case CODA_OP_UNFUSED_FWD: return unfused_fwd_ws(M, D);
    case CODA_OP_UNFUSED_BWD: return unfused_bwd_ws(M, D);
    case CODA_OP_FWD_SWIGLU: return (dim_ok(N) && N % 128 == 0) ? fwd_ws(M, D) : 0;
    case CODA_OP_BWD_SWIGLU: return (dim_ok(N) && N % 128 == 0) ? bwd_swiglu_ws(M, D, N) : 0;
    case CODA_OP_CE_FWD: return dim_ok(N) ? ce_fwd_ws(M, N) : 0;
    case CODA_OP_CE_BWD: return 0;
    case CODA_OP_UNFUSED_FWD_SWIGLU: return (dim_ok(N) && N % 128 == 0) ? fwd_ws(M, D) : 0;
    case CODA_OP_UNFUSED_BWD_SWIGLU: return (dim_ok(N) && N % 128 == 0) ? unfused_bwd_swiglu_ws(M, D, N) : 0;
    case CODA_OP_UNFUSED_CE_FWD:
    case CODA_OP_UNFUSED_CE_BWD: return dim_ok(N) ? unfused_ce_ws(M, N) : 0;
    default: break;
  }
  return 0;
}

coda_status_t coda_validate_fwd(const coda_fwd_args_t* a, const void* ws, size_t ws_bytes) {
  coda_status_t st = validate_fwd_common(a, true);
  if (st != CODA_OK) return st;
  return check_ws(ws, ws_bytes, fwd_ws(a->M, a->D));
}

coda_status_t coda_validate_fwd_noalloc(const coda_fwd_args_t* a) {
  coda_status_t st = validate_fwd_common(a, true);
  if (st != CODA_OK) return st;
  return fwd_ws_p(a->M, a->D) <= kNoAllocScratchBytes ? CODA_OK : CODA_ERR_WORKSPACE;
}

coda_status_t coda_validate_bwd(const coda_bwd_args_t* a, const void* ws, size_t ws_bytes) {
  coda_status_t st = validate_bwd_common(a);
  if (st != CODA_OK) return st;
  return check_ws(ws, ws_bytes, bwd_chain_ws(a->M, a->D, a->N));
}

// Used by the unfused entry point (g is optional there).
coda_status_t coda_validate_unfused(coda_op_t op, const void* args, const void* ws, size_t ws_bytes) {
  if (args == nullptr) return CODA_ERR_NULL;
  if (op == CODA_OP_FWD) {
    const coda_fwd_args_t* a = static_cast<const coda_fwd_args_t*>(args);
    coda_status_t st = validate_fwd_common(a, false);
    if (st != CODA_OK) return st;
    return check_ws(ws, ws_bytes, unfused_fwd_ws(a->M, a->D));
  }
  if (op == CODA_OP_BWD) {
    const coda_bwd_args_t* a = static_cast<const coda_bwd_args_t*>(args);
    coda_status_t st = validate_bwd_common(a);
    if (st != CODA_OK) return st;
    return check_ws(ws, ws_bytes, unfused_bwd_ws(a->M, a->D));
  }
  if (op == CODA_OP_FWD_SWIGLU)  // the fused chain forward's workspace
    return coda_validate_fwd_swiglu(static_cast<const coda_fwd_swiglu_args_t*>(args), ws, ws_bytes);
  if (op == CODA_OP_BWD_SWIGLU) {
    const coda_bwd_swiglu_args_t* a = static_cast<const coda_bwd_swiglu_args_t*>(args);
    coda_status_t st = validate_bwd_swiglu_common(a);
    if (st != CODA_OK) return st;
    return check_ws(ws, ws_bytes, unfused_bwd_swiglu_ws(a->M, a->D, a->N));
  }
  if (op == CODA_OP_CE_FWD) {
    const coda_ce_fwd_args_t* a = static_cast<const coda_ce_fwd_args_t*>(args);
    coda_status_t st = validate_ce_fwd_common(a);
    if (st != CODA_OK) return st;
    return check_ws(ws, ws_bytes, unfused_ce_ws(a->M, a->V));
  }
  if (op == CODA_OP_CE_BWD) {
    const coda_ce_bwd_args_t* a = static_cast<const coda_ce_bwd_args_t*>(args);
    coda_status_t st = coda_validate_ce_bwd(a);
    if (st != CODA_OK) return st;
    return check_ws(ws, ws_bytes, unfused_ce_ws(a->M, a->V));
  }
  return CODA_ERR_ARG;
}

coda_status_t coda_validate_gemm(const coda_gemm_args_t* a) {
  if (a == nullptr) return CODA_ERR_NULL;
  const void* ps[] = {a->A, a->B, a->C};
  coda_status_t st = check_ptrs(ps, 3);
  if (st != CODA_OK) return st;
  if (!rows_ok(a->M) || !dim_ok(a->N) || !dim_ok(a->K) || !grid_ok(a->M, a->N)) return CODA_ERR_SHAPE;
  if ((a->a_layout != CODA_ROW && a->a_layout != CODA_COL) ||
      (a->b_layout != CODA_ROW && a->b_layout != CODA_COL) || !dtype_ok(a->c_dtype))
    return CODA_ERR_ARG;
  const int64_t a_min = a->a_layout == CODA_ROW ? a->K : a->M;
  const int64_t b_min = a->b_layout == CODA_ROW ? a->N : a->K;
  if (a->lda < a_min || a->ldb < b_min || a->ldc < a->N) return CODA_ERR_SHAPE;
  if (a->lda % 8 || a->ldb % 8 || a->ldc % 8) return CODA_ERR_ALIGN;
  if (a->lda > kMaxDim || a->ldb > kMaxDim || a->ldc > kMaxDim) return CODA_ERR_SHAPE;
  return CODA_OK;
}

coda_status_t coda_validate_fwd_swiglu(const coda_fwd_swiglu_args_t* a, const void* ws, size_t ws_bytes) {
  if (a == nullptr) return CODA_ERR_NULL;
  coda_status_t st = coda_validate_fwd(&a->chain, ws, ws_bytes);
  if (st != CODA_OK) return st;
  const void* ps[] = {a->o};
  if ((st = check_ptrs(ps, 1)) != CODA_OK) return st;
  if (a->chain.N % 128) return CODA_ERR_SHAPE;
  if (a->chain.y_dtype != CODA_BF16 || !dtype_ok(a->o_dtype)) return CODA_ERR_ARG;
  return CODA_OK;
}

coda_status_t coda_validate_bwd_swiglu(const coda_bwd_swiglu_args_t* a, const void* ws, size_t ws_bytes) {
  coda_status_t st = validate_bwd_swiglu_common(a);
  if (st != CODA_OK) return st;
  return check_ws(ws, ws_bytes, bwd_swiglu_ws(a->M, a->D, a->N));
}

coda_status_t coda_validate_ce_fwd(const coda_ce_fwd_args_t* a, const void* ws, size_t ws_bytes) {
  coda_status_t st = validate_ce_fwd_common(a);
  if (st != CODA_OK) return st;
  return check_ws(ws, ws_bytes, ce_fwd_ws(a->M, a->V));
}

coda_status_t coda_validate_ce_bwd(const coda_ce_bwd_args_t* a) {
  if (a == nullptr) return CODA_ERR_NULL;
  const void* ps[] = {a->h, a->W, a->targets, a->lse, a->dloss, a->dlogits, a->dh, a->dW};
  coda_status_t st = check_ptrs(ps, 8);
  if (st != CODA_OK) return st;
  if (!rows_ok(a->M) || !dim_ok(a->D) || !dim_ok(a->V)) return CODA_ERR_SHAPE;
  if (!grid_ok(a->M, a->V) || !grid_ok(a->M, a->D) || !grid_ok(a->V, a->D)) return CODA_ERR_SHAPE;
  if (!dtype_ok(a->dh_dtype) || !dtype_ok(a->dW_dtype)) return CODA_ERR_ARG;
  if (a->logits != nullptr && !aligned16(a->logits)) return CODA_ERR_ALIGN;  // optional input
  return CODA_OK;
}

coda_status_t coda_validate_bwd_gemm0(const coda_bwd_gemm0_args_t* a) {
  if (a == nullptr) return CODA_ERR_NULL;
  const void* ps[] = {a->dh, a->x, a->W0, a->dx, a->dW0};
  coda_status_t st = check_ptrs(ps, 5);
  if (st != CODA_OK) return st;
  if (!rows_ok(a->M) || !dim_ok(a->K0) || !dim_ok(a->D)) return CODA_ERR_SHAPE;
  if (!grid_ok(a->M, a->K0) || !grid_ok(a->K0, a->D)) return CODA_ERR_SHAPE;
  if (!dtype_ok(a->dx_dtype) || !dtype_ok(a->dW0_dtype)) return CODA_ERR_ARG;
  return CODA_OK;
}

const char* coda_status_string(coda_status_t s) {
  switch (s) {
    case CODA_OK: return "ok";
    case CODA_ERR_NULL: return "a required pointer is NULL";
    case CODA_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case CODA_ERR_ALIGN: return "a pointer or leading dimension is not 16-byte aligned";
    case CODA_ERR_WORKSPACE: return "workspace missing or too small";
    case CODA_ERR_ARG: return "bad scalar argument";
    case CODA_ERR_HIP: return "HIP launch failed";
    default: break;
  }
  return "unknown status";
}

}  // extern "C"
