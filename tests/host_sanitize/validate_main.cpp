// Drives every host-side entry point of the C ABI (workspace sizes, argument validation, status
// strings) through valid and invalid arguments, for a build of coda_host.cpp with AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py). Pointers are fake aligned or
// misaligned addresses: validation never dereferences them. Exit status 0 means every call returned
// the expected status and no sanitizer fired (the sanitizers abort on the first finding).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <limits>

#include "coda.h"

namespace {

int failures = 0;

void expect(const char* what, coda_status_t got, coda_status_t want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, int(got), int(want));
    ++failures;
  }
}

void* fake(uintptr_t i) { return reinterpret_cast<void*>(0x100000 + 0x1000 * i); }
void* misaligned(uintptr_t i) { return reinterpret_cast<void*>(0x100000 + 0x1000 * i + 8); }

template <class E>
E raw(int v) {  // an enum field holding an arbitrary int, as a C caller may pass it
  E e;
  memcpy(&e, &v, sizeof e);
  return e;
}

const int64_t kBig[] = {0, -1, 1, 63, 64, 255, 256, 320, 4096, int64_t(1) << 20, (int64_t(1) << 20) + 64,
                        int64_t(1) << 22, (int64_t(1) << 22) + 1, int64_t(1) << 40,
                        std::numeric_limits<int64_t>::max(), std::numeric_limits<int64_t>::min()};

coda_fwd_args_t good_fwd() {
  coda_fwd_args_t a;
  memset(&a, 0, sizeof a);
  a.M = 300; a.K0 = 256; a.D = 512; a.N = 768; a.eps = 1e-5f;
  a.x = fake(1); a.W0 = fake(2); a.z = fake(3); a.gamma = fake(4); a.W1 = fake(5);
  a.h = fake(6); a.g = fake(7); a.r = static_cast<float*>(fake(8)); a.y = fake(9); a.y_dtype = CODA_BF16;
  return a;
}

coda_bwd_args_t good_bwd() {
  coda_bwd_args_t a;
  memset(&a, 0, sizeof a);
  a.M = 300; a.D = 512; a.N = 768;
  a.dY = fake(1); a.y = fake(2); a.h = fake(3); a.g = fake(4); a.r = static_cast<const float*>(fake(5));
  a.gamma = fake(6); a.W1 = fake(7); a.da = fake(8); a.dgamma = static_cast<float*>(fake(9)); a.dW1 = fake(10);
  a.s = static_cast<float*>(fake(11)); a.da_dtype = CODA_F32; a.dW1_dtype = CODA_BF16;
  return a;
}

}  // namespace

int main() {
  // workspace sizes over every op and extreme sizes: no overflow, no crash
  for (int op = -2; op < 14; ++op)
    for (int64_t M : kBig)
      for (int64_t D : kBig)
        for (int64_t N : kBig) (void)coda_workspace_bytes(raw<coda_op_t>(op), M, D, N);

  const size_t big_ws = size_t(1) << 40;
  {
    coda_fwd_args_t a = good_fwd();
    expect("fwd ok", coda_validate_fwd(&a, fake(20), big_ws), CODA_OK);
    expect("fwd null args", coda_validate_fwd(nullptr, fake(20), big_ws), CODA_ERR_NULL);
    a.z = nullptr;
    expect("fwd null z", coda_validate_fwd(&a, fake(20), big_ws), CODA_ERR_NULL);
    a = good_fwd(); a.W1 = misaligned(5);
    expect("fwd misaligned W1", coda_validate_fwd(&a, fake(20), big_ws), CODA_ERR_ALIGN);
    a = good_fwd();
    expect("fwd no workspace", coda_validate_fwd(&a, nullptr, 0), CODA_ERR_WORKSPACE);
    expect("fwd small workspace", coda_validate_fwd(&a, fake(20), 16), CODA_ERR_WORKSPACE);
    expect("fwd misaligned workspace", coda_validate_fwd(&a, misaligned(20), big_ws), CODA_ERR_ALIGN);
    for (int64_t v : kBig) {
      a = good_fwd(); a.M = v; (void)coda_validate_fwd(&a, fake(20), big_ws);
      a = good_fwd(); a.K0 = v; (void)coda_validate_fwd(&a, fake(20), big_ws);
      a = good_fwd(); a.D = v; (void)coda_validate_fwd(&a, fake(20), big_ws);
      a = good_fwd(); a.N = v; (void)coda_validate_fwd(&a, fake(20), big_ws);
    }
    const float bad_eps[] = {0.0f, -1e-5f, std::numeric_limits<float>::quiet_NaN(),
                             std::numeric_limits<float>::infinity()};
    for (float e : bad_eps) {
      a = good_fwd(); a.eps = e;
      expect("fwd bad eps", coda_validate_fwd(&a, fake(20), big_ws), CODA_ERR_ARG);
    }
    a = good_fwd();
    expect("fwd_noalloc ok", coda_validate_fwd_noalloc(&a), CODA_OK);
    a.M = int64_t(1) << 22; a.D = 4096;     // partials of 2^22 x 64 fp32 = 1 GiB > the 16 MiB scratch
    expect("fwd_noalloc too large", coda_validate_fwd_noalloc(&a), CODA_ERR_WORKSPACE);
    expect("fwd_noalloc null", coda_validate_fwd_noalloc(nullptr), CODA_ERR_NULL);
    for (int t : {-1, 2, 7, 1 << 30}) {
      a = good_fwd(); a.y_dtype = raw<coda_dtype_t>(t);
      expect("fwd bad dtype", coda_validate_fwd(&a, fake(20), big_ws), CODA_ERR_ARG);
    }
    // every op code against an argument block as large as any args struct (the op decides its type)
    union {
      coda_fwd_args_t f;
      coda_bwd_args_t b;
      coda_fwd_swiglu_args_t fs;
      coda_bwd_swiglu_args_t bs;
      coda_ce_fwd_args_t cf;
      coda_ce_bwd_args_t cb;
    } any;
    memset(&any, 0, sizeof any);
    any.f = good_fwd();
    for (int op = -2; op < 14; ++op) (void)coda_validate_unfused(raw<coda_op_t>(op), &any, fake(20), big_ws);
    expect("unfused fwd ok", coda_validate_unfused(CODA_OP_FWD, &any, fake(20), big_ws), CODA_OK);
    expect("unfused null", coda_validate_unfused(CODA_OP_FWD, nullptr, fake(20), big_ws), CODA_ERR_NULL);
  }
  {
    coda_bwd_args_t a = good_bwd();
    expect("bwd ok", coda_validate_bwd(&a, fake(20), big_ws), CODA_OK);
    expect("bwd null args", coda_validate_bwd(nullptr, fake(20), big_ws), CODA_ERR_NULL);
    a.s = nullptr;
    expect("bwd null s", coda_validate_bwd(&a, fake(20), big_ws), CODA_ERR_NULL);
    for (int64_t v : kBig) {
      a = good_bwd(); a.M = v; (void)coda_validate_bwd(&a, fake(20), big_ws);
      a = good_bwd(); a.D = v; (void)coda_validate_bwd(&a, fake(20), big_ws);
      a = good_bwd(); a.N = v; (void)coda_validate_bwd(&a, fake(20), big_ws);
    }
    for (int t : {-1, 2, 1 << 30}) {
      a = good_bwd(); a.dW1_dtype = raw<coda_dtype_t>(t);
      expect("bwd bad dtype", coda_validate_bwd(&a, fake(20), big_ws), CODA_ERR_ARG);
    }
  }
  {
    coda_gemm_args_t g;
    memset(&g, 0, sizeof g);
    g.M = 300; g.N = 512; g.K = 768; g.A = fake(1); g.lda = 768; g.a_layout = CODA_ROW;
    g.B = fake(2); g.ldb = 512; g.b_layout = CODA_ROW; g.C = fake(3); g.ldc = 512; g.c_dtype = CODA_F32;
    expect("gemm ok", coda_validate_gemm(&g), CODA_OK);
    for (int64_t v : kBig) {
      coda_gemm_args_t h = g; h.M = v; (void)coda_validate_gemm(&h);
      h = g; h.lda = v; (void)coda_validate_gemm(&h);
      h = g; h.ldb = v; (void)coda_validate_gemm(&h);
      h = g; h.ldc = v; (void)coda_validate_gemm(&h);
      h = g; h.K = v; (void)coda_validate_gemm(&h);
    }
    coda_gemm_args_t h = g;
    h.a_layout = raw<coda_layout_t>(5);
    expect("gemm bad layout", coda_validate_gemm(&h), CODA_ERR_ARG);
  }
  {
    coda_bwd_gemm0_args_t b;
    memset(&b, 0, sizeof b);
    b.M = 300; b.K0 = 256; b.D = 512; b.dh = fake(1); b.x = fake(2); b.W0 = fake(3); b.dx = fake(4); b.dW0 = fake(5);
    expect("bwd_gemm0 ok", coda_validate_bwd_gemm0(&b), CODA_OK);
    for (int64_t v : kBig) {
      coda_bwd_gemm0_args_t c = b; c.M = v; (void)coda_validate_bwd_gemm0(&c);
      c = b; c.K0 = v; (void)coda_validate_bwd_gemm0(&c);
    }
  }
  {
    coda_fwd_swiglu_args_t s;
    memset(&s, 0, sizeof s);
    s.chain = good_fwd(); s.chain.N = 1024; s.o = fake(12); s.o_dtype = CODA_F32;
    expect("fwd_swiglu ok", coda_validate_fwd_swiglu(&s, fake(20), big_ws), CODA_OK);
    coda_bwd_swiglu_args_t b;
    memset(&b, 0, sizeof b);
    b.M = 300; b.D = 512; b.N = 1024; b.E = 256;
    const void* ps[] = {fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7), fake(8), fake(9)};
    b.dOut = ps[0]; b.W2 = ps[1]; b.o = ps[2]; b.y = ps[3]; b.h = ps[4]; b.g = ps[5];
    b.r = static_cast<const float*>(ps[6]); b.gamma = ps[7]; b.W1 = ps[8];
    b.dY = fake(10); b.da = fake(11); b.dgamma = static_cast<float*>(fake(12)); b.dW1 = fake(13); b.dW2 = fake(14);
    b.s = static_cast<float*>(fake(15));
    expect("bwd_swiglu ok", coda_validate_bwd_swiglu(&b, fake(20), big_ws), CODA_OK);
    for (int64_t v : kBig) {
      coda_bwd_swiglu_args_t c = b; c.E = v; (void)coda_validate_bwd_swiglu(&c, fake(20), big_ws);
      c = b; c.N = v; (void)coda_validate_bwd_swiglu(&c, fake(20), big_ws);
    }
  }
  {
    coda_ce_fwd_args_t f;
    memset(&f, 0, sizeof f);
    f.M = 300; f.D = 512; f.V = 1024; f.h = fake(1); f.W = fake(2);
    f.targets = static_cast<const int64_t*>(fake(3)); f.lse = static_cast<float*>(fake(4));
    f.loss = static_cast<float*>(fake(5));
    expect("ce_fwd ok", coda_validate_ce_fwd(&f, fake(20), big_ws), CODA_OK);
    f.logits = static_cast<float*>(misaligned(6));
    expect("ce_fwd misaligned logits", coda_validate_ce_fwd(&f, fake(20), big_ws), CODA_ERR_ALIGN);
    coda_ce_bwd_args_t b;
    memset(&b, 0, sizeof b);
    b.M = 300; b.D = 512; b.V = 1024; b.h = fake(1); b.W = fake(2); b.targets = static_cast<const int64_t*>(fake(3));
    b.lse = static_cast<const float*>(fake(4)); b.dloss = static_cast<const float*>(fake(5)); b.dlogits = fake(6);
    b.dh = fake(7); b.dW = fake(8);
    expect("ce_bwd ok", coda_validate_ce_bwd(&b), CODA_OK);
    for (int64_t v : kBig) {
      coda_ce_bwd_args_t c = b; c.V = v; (void)coda_validate_ce_bwd(&c);
    }
  }
  for (int s = -3; s < 10; ++s) {
    const char* str = coda_status_string(raw<coda_status_t>(s));
    if (str == nullptr || strlen(str) == 0) ++failures;
  }
  if (failures) {
    fprintf(stderr, "%d unexpected status(es)\n", failures);
    return 1;
  }
  printf("host validation under sanitizers: ok\n");
  return 0;
}
