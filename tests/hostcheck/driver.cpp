// Host-side checks of the libdspark C ABI (csrc/api.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer: every entry point with valid arguments
// reaches its launcher with exactly those arguments, and with invalid ones
// returns the documented status without calling it.  No pointer passed here
// is ever dereferenced: the ABI validates and forwards them only.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "dspark.h"
#include "hostcheck.hpp"

using hostcheck::last;

static int failures = 0;

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);   \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static void* P(uintptr_t x) { return reinterpret_cast<void*>(x); }
static const uintptr_t A = 0x10000, Bp = 0x20000, C = 0x30000, D = 0x40000, E = 0x50000, F = 0x60000,
                       G = 0x70000, H = 0x80000, I = 0x90000, J = 0xA0000, K = 0xB0000, L = 0xC0000;

static void reset() { memset(&last, 0, sizeof(last)); }

static dspark_status draft(int B, int gamma, int V, int r, float T, const void* W2T, size_t wsb, uintptr_t U = A,
                           uintptr_t x0 = D) {
  return dspark_markov_draft((const float*)P(U), P(Bp), P(C), W2T, DSPARK_BF16, (const int32_t*)P(x0), B, gamma, V,
                             r, T, (const uint64_t*)P(E), 42, (int32_t*)P(F), (float*)P(G), (float*)P(H), nullptr,
                             nullptr, nullptr, 0, nullptr, P(I), wsb, nullptr);
}

int main() {
  // version, status strings (every code, and an unknown one)
  CHECK(dspark_version() >= 100);
  for (int s = -5; s <= 0; ++s) CHECK(strlen(dspark_status_string((dspark_status)s)) > 1);
  CHECK(strcmp(dspark_status_string((dspark_status)99), "unknown status") == 0);

  // workspace sizes: 0 out of range, positive in range
  CHECK(dspark_workspace_size(DSPARK_OP_DRAFT, 0, 4, 1000, 16) == 0);
  CHECK(dspark_workspace_size(DSPARK_OP_DRAFT, 4, 33, 1000, 16) == 0);
  CHECK(dspark_workspace_size(DSPARK_OP_DRAFT, 4, 4, 1, 16) == 0);
  CHECK(dspark_workspace_size(DSPARK_OP_DRAFT, 4, 4, 1000, 24) == 0);
  CHECK(dspark_workspace_size(DSPARK_OP_DRAFT, 65537, 4, 1000, 16) == 0);
  CHECK(dspark_workspace_size((dspark_op)9, 4, 4, 1000, 16) == 0);
  for (int op = 0; op < 4; ++op) CHECK(dspark_workspace_size((dspark_op)op, 256, 7, 151936, 256) > 0);
  // the largest sizes: no overflow in the size arithmetic
  CHECK(dspark_workspace_size(DSPARK_OP_VERIFY, 65536, 32, 2147483647, 512) > (size_t)1 << 40);

  // draft: valid call forwards every argument
  const size_t wsd = dspark_workspace_size(DSPARK_OP_DRAFT, 256, 7, 151936, 256);
  reset();
  CHECK(draft(256, 7, 151936, 256, 0.7f, P(J), wsd) == DSPARK_OK);
  CHECK(strcmp(last.op, "draft") == 0 && last.B == 256 && last.gamma == 7 && last.V == 151936 && last.r == 256);
  CHECK(last.T == 0.7f && last.round == 42 && last.bf16 && last.ws == P(I) && last.suppressed == 0);
  CHECK(last.p[0] == P(A) && last.p[1] == P(Bp) && last.p[2] == P(C) && last.p[3] == P(J) && last.p[4] == P(D));
  CHECK(last.p[5] == P(E) && last.p[6] == P(F) && last.p[7] == P(G) && last.p[8] == P(H) && last.p[9] == nullptr);
  // the confidence head: forwarded with its output; its inputs are not read
  // (not even checked) without one
  reset();
  CHECK(dspark_markov_draft((const float*)P(A), P(Bp), P(C), nullptr, DSPARK_BF16, (const int32_t*)P(D), 8, 4, 1000,
                            16, 1.0f, (const uint64_t*)P(E), 0, (int32_t*)P(F), (float*)P(G), (float*)P(H),
                            (const float*)P(K), (const float*)P(L), nullptr, 4096, (float*)P(J), P(I), 1 << 30,
                            nullptr) == DSPARK_OK);
  CHECK(last.p[9] == P(J) && last.d == 4096);
  reset();
  CHECK(dspark_markov_draft((const float*)P(A), P(Bp), P(C), nullptr, DSPARK_BF16, (const int32_t*)P(D), 8, 4, 1000,
                            16, 1.0f, (const uint64_t*)P(E), 0, (int32_t*)P(F), (float*)P(G), (float*)P(H),
                            (const float*)P(K + 4), nullptr, nullptr, -3, nullptr, P(I), 1 << 30,
                            nullptr) == DSPARK_OK);
  CHECK(last.p[9] == nullptr && last.d == 0);
  reset();
  CHECK(dspark_markov_draft((const float*)P(A), P(Bp), P(C), nullptr, DSPARK_BF16, (const int32_t*)P(D), 8, 4, 1000,
                            16, 1.0f, (const uint64_t*)P(E), 0, (int32_t*)P(F), (float*)P(G), (float*)P(H),
                            (const float*)P(K + 4), (const float*)P(L), nullptr, 4096, (float*)P(J), P(I), 1 << 30,
                            nullptr) == DSPARK_ERR_INVALID_ARGUMENT);
  CHECK(last.op[0] == 0);
  // draft: each bad argument returns its status and launches nothing
  struct Bad {
    int B, gamma, V, r;
    float T;
    const void* W2T;
    size_t wsb;
    uintptr_t U, x0;
    dspark_status want;
  } bad[] = {
      {0, 7, 1000, 16, 1.0f, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 0, 1000, 16, 1.0f, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 33, 1000, 16, 1.0f, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, 1, 16, 1.0f, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, 1000, 8, 1.0f, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, 1000, 520, 1.0f, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, 1000, 16, -0.5f, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, 1000, 16, NAN, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, 1000, 16, INFINITY, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, 1000, 16, 1.0f, nullptr, 1 << 30, 0, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, 1000, 16, 1.0f, nullptr, 1 << 30, A + 4, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, 1000, 16, 1.0f, nullptr, 1 << 30, A, D + 2, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, 1000, 16, 1.0f, P(C), 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},     // W2T aliases W2
      {4, 4, 1000, 16, 1.0f, P(J + 8), 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},  // W2T misaligned
      {4, 4, 1000, 16, 1.0f, nullptr, 16, A, D, DSPARK_ERR_WORKSPACE},
      {2147483647, 4, 1000, 16, 1.0f, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
      {4, 4, -5, 16, 1.0f, nullptr, 1 << 30, A, D, DSPARK_ERR_INVALID_ARGUMENT},
  };
  for (const Bad& b : bad) {
    reset();
    CHECK(draft(b.B, b.gamma, b.V, b.r, b.T, b.W2T, b.wsb, b.U, b.x0) == b.want);
    CHECK(last.op[0] == 0);
  }
  reset();
  CHECK(dspark_markov_draft((const float*)P(A), P(Bp), P(C), nullptr, (dspark_dtype)7, (const int32_t*)P(D), 4, 4,
                            1000, 16, 1.0f, (const uint64_t*)P(E), 0, (int32_t*)P(F), (float*)P(G), (float*)P(H),
                            nullptr, nullptr, nullptr, 0, nullptr, P(I), 1 << 30, nullptr) == DSPARK_ERR_UNSUPPORTED);
  // T == 0 needs no seeds
  reset();
  CHECK(dspark_markov_draft((const float*)P(A), P(Bp), P(C), nullptr, DSPARK_BF16, (const int32_t*)P(D), 4, 4, 1000,
                            16, 0.0f, nullptr, 0, (int32_t*)P(F), (float*)P(G), (float*)P(H), nullptr, nullptr,
                            nullptr, 0, nullptr, P(I), 1 << 30, nullptr) == DSPARK_OK);
  CHECK(strcmp(last.op, "draft") == 0 && last.p[5] == nullptr);

  // allocation-free draft: the static array, profiling suppressed, size limit
  reset();
  CHECK(dspark_markov_draft_noalloc((const float*)P(A), P(Bp), P(C), P(J), DSPARK_BF16, (const int32_t*)P(D), 256, 7,
                                    151936, 256, 1.0f, (const uint64_t*)P(E), 3, (int32_t*)P(F), (float*)P(G),
                                    (float*)P(H), nullptr, nullptr, nullptr, 0, nullptr, nullptr) == DSPARK_OK);
  CHECK(strcmp(last.op, "draft") == 0 && last.ws != nullptr && last.suppressed == 1 && last.p[3] == P(J));
  reset();
  CHECK(dspark_markov_draft_noalloc((const float*)P(A), P(Bp), P(C), nullptr, DSPARK_BF16, (const int32_t*)P(D),
                                    65536, 32, 1 << 20, 256, 1.0f, (const uint64_t*)P(E), 3, (int32_t*)P(F),
                                    (float*)P(G), (float*)P(H), nullptr, nullptr, nullptr, 0, nullptr,
                                    nullptr) == DSPARK_ERR_SCRATCH_LIMIT);
  CHECK(last.op[0] == 0);
  CHECK(dspark_static_scratch_bytes() == (size_t)32 << 20);

  // verify: valid, lengths and W2T forwarded; greedy needs neither U nor seeds
  const size_t wsv = dspark_workspace_size(DSPARK_OP_VERIFY, 8, 4, 5000, 64);
  reset();
  CHECK(dspark_verify((const float*)P(A), P(Bp), P(C), P(J), DSPARK_BF16, (const int32_t*)P(D), (const int32_t*)P(F),
                      (const float*)P(G), nullptr, (const float*)P(K), (const int32_t*)P(L), 8, 4, 5000, 64, 1.0f,
                      (const uint64_t*)P(E), 5, (int32_t*)P(H), (int32_t*)P(I), (float*)P(A + 0x1000), P(0xD0000), wsv,
                      nullptr) == DSPARK_OK);
  CHECK(strcmp(last.op, "verify") == 0 && last.p[1] == P(J) && last.p[2] == P(K) && last.p[3] == P(L) &&
        last.p[5] == nullptr);
  reset();
  CHECK(dspark_verify((const float*)P(A), P(Bp), P(C), nullptr, DSPARK_BF16, (const int32_t*)P(D),
                      (const int32_t*)P(F), (const float*)P(G), (const float*)P(A + 0x2000), (const float*)P(K),
                      nullptr, 8, 4, 5000, 64, 1.0f, (const uint64_t*)P(E), 5, (int32_t*)P(H), (int32_t*)P(I), nullptr,
                      P(0xD0000), wsv, nullptr) == DSPARK_OK);
  CHECK(last.p[5] == P(A + 0x2000));  // the RNN draft's operand rows
  reset();
  CHECK(dspark_verify(nullptr, nullptr, nullptr, nullptr, DSPARK_BF16, (const int32_t*)P(D), (const int32_t*)P(F),
                      nullptr, nullptr, (const float*)P(K), nullptr, 8, 4, 5000, 64, 0.0f, nullptr, 5, (int32_t*)P(H),
                      (int32_t*)P(I), nullptr, P(0xD0000), wsv, nullptr) == DSPARK_OK);
  CHECK(last.p[1] == nullptr);  // no W2T at T == 0
  reset();
  CHECK(dspark_verify(nullptr, nullptr, nullptr, nullptr, DSPARK_BF16, (const int32_t*)P(D), (const int32_t*)P(F),
                      nullptr, nullptr, (const float*)P(K), nullptr, 8, 4, 5000, 64, 1.0f, nullptr, 5, (int32_t*)P(H),
                      (int32_t*)P(I), nullptr, P(0xD0000), wsv, nullptr) == DSPARK_ERR_INVALID_ARGUMENT);
  CHECK(last.op[0] == 0);
  reset();
  CHECK(dspark_verify((const float*)P(A), P(Bp), P(C), nullptr, DSPARK_BF16, (const int32_t*)P(D),
                      (const int32_t*)P(F), (const float*)P(G), nullptr, (const float*)P(K), nullptr, 8, 4, 5000, 64,
                      1.0f, (const uint64_t*)P(E), 5, (int32_t*)P(H), (int32_t*)P(I), nullptr, P(0xD0000), wsv - 1,
                      nullptr) == DSPARK_ERR_WORKSPACE);

  // survival: confidence mode needs nothing else; analytical mode validates
  reset();
  CHECK(dspark_survival(nullptr, nullptr, nullptr, DSPARK_BF16, nullptr, nullptr, nullptr, nullptr, nullptr,
                        (const float*)P(A), 8, 4, 2, 16, 0.0f, nullptr, (float*)P(Bp), nullptr, 0, nullptr) ==
        DSPARK_OK);
  CHECK(strcmp(last.op, "survival_conf") == 0 && last.p[0] == P(A) && last.p[1] == P(Bp));
  reset();
  CHECK(dspark_survival(nullptr, nullptr, nullptr, DSPARK_BF16, nullptr, nullptr, nullptr, nullptr, nullptr,
                        (const float*)P(A + 2), 8, 4, 2, 16, 0.0f, nullptr, (float*)P(Bp), nullptr, 0, nullptr) ==
        DSPARK_ERR_INVALID_ARGUMENT);
  CHECK(dspark_survival(nullptr, nullptr, nullptr, DSPARK_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        8, 4, 5000, 64, 1.0f, nullptr, (float*)P(Bp), P(C), 1 << 30, nullptr) ==
        DSPARK_ERR_INVALID_ARGUMENT);
  // analytical mode forwards the RNN draft's operand rows
  reset();
  CHECK(dspark_survival((const float*)P(A), P(Bp), P(C), DSPARK_BF16, (const int32_t*)P(D), (const int32_t*)P(F),
                        (const float*)P(G), (const float*)P(A + 0x2000), (const float*)P(K), nullptr, 8, 4, 5000, 64,
                        1.0f, nullptr, (float*)P(H), P(0xD0000), dspark_workspace_size(DSPARK_OP_SURVIVAL, 8, 4, 5000,
                        64), nullptr) == DSPARK_OK);
  CHECK(strcmp(last.op, "survival") == 0 && last.p[3] == P(A + 0x2000));

  // schedule: candidate limit, table length, modes
  reset();
  CHECK(dspark_schedule((const float*)P(A), (const double*)P(Bp), 1 << 20, 2048, 8, DSPARK_SCHEDULE_EARLY_STOP,
                        nullptr, nullptr, (int32_t*)P(C), nullptr, nullptr) == DSPARK_OK);  // 16384 candidates
  reset();
  CHECK(dspark_schedule((const float*)P(A), (const double*)P(Bp), 256 * 8 + 1, 256, 7, DSPARK_SCHEDULE_EARLY_STOP,
                        nullptr, nullptr, (int32_t*)P(C), nullptr, nullptr) == DSPARK_OK);
  CHECK(strcmp(last.op, "schedule") == 0 && last.B == 256 && last.mode == 0);
  CHECK(dspark_schedule((const float*)P(A), (const double*)P(Bp), 256 * 8, 256, 7, DSPARK_SCHEDULE_EARLY_STOP,
                        nullptr, nullptr, (int32_t*)P(C), nullptr, nullptr) == DSPARK_ERR_INVALID_ARGUMENT);
  CHECK(dspark_schedule((const float*)P(A), (const double*)P(Bp), 1 << 20, 16385, 1, DSPARK_SCHEDULE_EARLY_STOP,
                        nullptr, nullptr, (int32_t*)P(C), nullptr, nullptr) == DSPARK_ERR_INVALID_ARGUMENT);
  CHECK(dspark_schedule((const float*)P(A), (const double*)P(Bp), 1 << 20, 16, 4, DSPARK_SCHEDULE_TOP_K, nullptr,
                        nullptr, (int32_t*)P(C), nullptr, nullptr) == DSPARK_ERR_INVALID_ARGUMENT);
  CHECK(dspark_schedule((const float*)P(A), (const double*)P(Bp), 1 << 20, 16, 4, (dspark_schedule_mode)3, nullptr,
                        nullptr, (int32_t*)P(C), nullptr, nullptr) == DSPARK_ERR_INVALID_ARGUMENT);
  // a capacity output is only written in capacity mode
  reset();
  CHECK(dspark_schedule((const float*)P(A), (const double*)P(Bp), 1 << 20, 16, 4, DSPARK_SCHEDULE_EARLY_STOP,
                        nullptr, (int32_t*)P(D), (int32_t*)P(C), nullptr, nullptr) == DSPARK_OK);
  CHECK(last.p[1] == nullptr);

  // confidence, transpose, bias
  reset();
  CHECK(dspark_confidence((const float*)P(A), (const float*)P(Bp), P(C), DSPARK_BF16, (const int32_t*)P(D),
                          (const int32_t*)P(E), nullptr, 8, 4, 4096, 5000, 64, (float*)P(F), nullptr) == DSPARK_OK);
  CHECK(strcmp(last.op, "confidence") == 0 && last.d == 4096);
  CHECK(dspark_confidence((const float*)P(A), (const float*)P(Bp), P(C), DSPARK_BF16, (const int32_t*)P(D),
                          (const int32_t*)P(E), nullptr, 8, 4, (1 << 20) + 1, 5000, 64, (float*)P(F), nullptr) ==
        DSPARK_ERR_INVALID_ARGUMENT);
  CHECK(dspark_transpose_w2(P(A), DSPARK_BF16, 256, 151936, P(A), nullptr) == DSPARK_ERR_INVALID_ARGUMENT);
  reset();
  CHECK(dspark_transpose_w2(P(A), DSPARK_BF16, 256, 151936, P(Bp), nullptr) == DSPARK_OK);
  CHECK(strcmp(last.op, "transpose_w2") == 0 && last.V == 151936);
  CHECK(dspark_markov_bias(P(A), P(Bp), DSPARK_F32, (const int32_t*)P(C), (1 << 20) + 1, 1000, 16, (float*)P(D),
                           nullptr) == DSPARK_ERR_INVALID_ARGUMENT);

  // RNN draft: bf16 only
  const size_t wsr = dspark_workspace_size(DSPARK_OP_RNN_DRAFT, 8, 4, 5000, 64);
  reset();
  CHECK(dspark_rnn_draft((const float*)P(A), P(Bp), P(C), DSPARK_BF16, (const float*)P(D), (const float*)P(E),
                         (const int32_t*)P(F), 8, 4, 5000, 64, 1.0f, (const uint64_t*)P(G), 0, (int32_t*)P(H),
                         (float*)P(I), (float*)P(J), nullptr, P(K), wsr, nullptr) == DSPARK_OK);
  CHECK(strcmp(last.op, "rnn_draft") == 0 && last.p[3] == nullptr);
  CHECK(dspark_rnn_draft((const float*)P(A), P(Bp), P(C), DSPARK_F32, (const float*)P(D), (const float*)P(E),
                         (const int32_t*)P(F), 8, 4, 5000, 64, 1.0f, (const uint64_t*)P(G), 0, (int32_t*)P(H),
                         (float*)P(I), (float*)P(J), nullptr, P(K), wsr, nullptr) == DSPARK_ERR_UNSUPPORTED);

  if (failures) {
    fprintf(stderr, "%d host checks failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
