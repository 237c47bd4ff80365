// The libdspark C ABI: argument validation (host only, before any HIP call),
// workspace sizing and dispatch to the kernel launchers.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "dspark.h"
#include "launch.hpp"

using namespace dspark;

namespace {

constexpr int kMaxB = 65536;
constexpr int kMaxGamma = 32;
constexpr int kMaxR = 512;

bool sizes_ok(int B, int gamma, int V, int r) {
  return B >= 1 && B <= kMaxB && gamma >= 1 && gamma <= kMaxGamma && V >= 2 && r >= 16 && r <= kMaxR &&
         r % 16 == 0;
}

bool temp_ok(float T) { return isfinite(T) && T >= 0.0f; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A required pointer: non-null and aligned.
bool req(const void* p, size_t a) { return p != nullptr && aligned(p, a); }

// An optional pointer: null, or aligned.
bool opt(const void* p, size_t a) { return p == nullptr || aligned(p, a); }

// The integer a caller passed for an enum parameter.  A C caller may pass any
// int there, and in C++ reading an enum object whose value lies outside the
// range of its enumerators is undefined, so every enum argument is first
// read through its bytes and range-checked as an int.
template <class E>
int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "the enums of the C ABI are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

bool dtype_ok(int d) { return d == DSPARK_F32 || d == DSPARK_BF16; }

// The optional confidence head of dspark_markov_draft: conf == null, or its
// inputs present, aligned and sized.
bool conf_head_ok(const float* h, const float* w, const float* sts, int d, const float* conf) {
  if (conf == nullptr) return true;
  return aligned(conf, 4) && req(h, 16) && req(w, 16) && opt(sts, 4) && d >= 1 && d <= (1 << 20);
}

dspark_status from_hip(hipError_t e) { return e == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP; }

}  // namespace

extern "C" {

int dspark_version(void) { return 100; }

const char* dspark_status_string(dspark_status status) {
  switch (enum_value(status)) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DSPARK_ERR_UNSUPPORTED: return "unsupported weight dtype";
    case DSPARK_ERR_WORKSPACE: return "workspace too small";
    case DSPARK_ERR_HIP: return "HIP launch error";
    case DSPARK_ERR_SCRATCH_LIMIT: return "sizes exceed the static scratch array of the allocation-free entry point";
    default: return "unknown status";
  }
}

size_t dspark_workspace_size(dspark_op op_arg, int B, int gamma, int V, int r) {
  if (!sizes_ok(B, gamma, V, r)) return 0;
  switch (enum_value(op_arg)) {
    case DSPARK_OP_DRAFT: return draft_workspace(B, gamma, V, r);
    case DSPARK_OP_VERIFY: return verify_workspace(B, gamma, V, r);
    case DSPARK_OP_SURVIVAL: return survival_workspace(B, gamma, V, r);
    case DSPARK_OP_RNN_DRAFT: return rnn_draft_workspace(B, gamma, V, r);
    default: return 0;
  }
}

dspark_status dspark_markov_bias(const void* W1, const void* W2, dspark_dtype wdtype, const int32_t* tokens,
                                 int n, int V, int r, float* out, hipStream_t stream) {
  if (!dtype_ok(enum_value(wdtype))) return DSPARK_ERR_UNSUPPORTED;
  if (!sizes_ok(1, 1, V, r) || n < 1 || n > (1 << 20)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!req(W1, 16) || !req(W2, 16) || !req(tokens, 4) || !req(out, 4)) return DSPARK_ERR_INVALID_ARGUMENT;
  return from_hip(launch_markov_bias(W1, W2, wdtype == DSPARK_BF16, tokens, n, V, r, out, stream));
}

dspark_status dspark_markov_draft(const float* U, const void* W1, const void* W2, const void* W2T,
                                  dspark_dtype wdtype, const int32_t* x0, int B, int gamma, int V, int r,
                                  float temperature,
                                  const uint64_t* seeds, uint64_t round, int32_t* draft_tokens, float* draft_prob,
                                  float* draft_lse, const float* conf_h, const float* conf_w, const float* conf_sts,
                                  int conf_d, float* conf, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (!dtype_ok(enum_value(wdtype))) return DSPARK_ERR_UNSUPPORTED;
  if (!sizes_ok(B, gamma, V, r) || !temp_ok(temperature)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!req(U, 16) || !req(W1, 16) || !req(W2, 16) || !opt(W2T, 16) || W2T == W2 || !req(x0, 4) ||
      !req(draft_tokens, 4) || !req(draft_prob, 4) || !req(draft_lse, 4) || !req(workspace, 16) ||
      !conf_head_ok(conf_h, conf_w, conf_sts, conf_d, conf))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (temperature > 0.0f && !req(seeds, 8)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < draft_workspace(B, gamma, V, r)) return DSPARK_ERR_WORKSPACE;
  DraftArgs a = {};
  a.U = U;
  a.W1 = W1;
  a.W2 = W2;
  a.W2T = W2T;
  a.x0 = x0;
  a.seeds = seeds;
  a.round = round;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.r = r;
  a.temperature = temperature;
  a.tokens = draft_tokens;
  a.prob = draft_prob;
  a.lse = draft_lse;
  if (conf) {
    a.ch = conf_h;
    a.cw = conf_w;
    a.csts = conf_sts;
    a.cd = conf_d;
    a.conf = conf;
  }
  a.ws = workspace;
  return from_hip(launch_draft(a, wdtype == DSPARK_BF16, stream));
}

dspark_status dspark_markov_draft_noalloc(const float* U, const void* W1, const void* W2, const void* W2T,
                                          dspark_dtype wdtype, const int32_t* x0, int B, int gamma, int V, int r,
                                          float temperature,
                                          const uint64_t* seeds, uint64_t round, int32_t* draft_tokens,
                                          float* draft_prob, float* draft_lse, const float* conf_h,
                                          const float* conf_w, const float* conf_sts, int conf_d, float* conf,
                                          hipStream_t stream) {
  if (!dtype_ok(enum_value(wdtype))) return DSPARK_ERR_UNSUPPORTED;
  if (!sizes_ok(B, gamma, V, r) || !temp_ok(temperature)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!req(U, 16) || !req(W1, 16) || !req(W2, 16) || !opt(W2T, 16) || W2T == W2 || !req(x0, 4) ||
      !req(draft_tokens, 4) || !req(draft_prob, 4) || !req(draft_lse, 4) ||
      !conf_head_ok(conf_h, conf_w, conf_sts, conf_d, conf))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (temperature > 0.0f && !req(seeds, 8)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (draft_workspace(B, gamma, V, r) > static_scratch_bytes()) return DSPARK_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (static_scratch(&ws) != hipSuccess) return DSPARK_ERR_HIP;
  ProfSuppress quiet;
  DraftArgs a = {};
  a.U = U;
  a.W1 = W1;
  a.W2 = W2;
  a.W2T = W2T;
  a.x0 = x0;
  a.seeds = seeds;
  a.round = round;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.r = r;
  a.temperature = temperature;
  a.tokens = draft_tokens;
  a.prob = draft_prob;
  a.lse = draft_lse;
  if (conf) {
    a.ch = conf_h;
    a.cw = conf_w;
    a.csts = conf_sts;
    a.cd = conf_d;
    a.conf = conf;
  }
  a.ws = ws;
  return from_hip(launch_draft(a, wdtype == DSPARK_BF16, stream));
}

size_t dspark_static_scratch_bytes(void) { return static_scratch_bytes(); }

dspark_status dspark_rnn_draft(const float* U, const void* W1, const void* W2, dspark_dtype wdtype,
                               const float* Wp, const float* hp, const int32_t* x0, int B, int gamma, int V, int r,
                               float temperature, const uint64_t* seeds, uint64_t round, int32_t* draft_tokens,
                               float* draft_prob, float* draft_lse, float* e_out, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  if (enum_value(wdtype) != DSPARK_BF16) return DSPARK_ERR_UNSUPPORTED;
  if (!sizes_ok(B, gamma, V, r) || !temp_ok(temperature)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!req(U, 16) || !req(W1, 16) || !req(W2, 16) || !req(Wp, 16) || !req(hp, 4) || !req(x0, 4) ||
      !req(draft_tokens, 4) || !req(draft_prob, 4) || !req(draft_lse, 4) || !opt(e_out, 4) ||
      !req(workspace, 16))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (temperature > 0.0f && !req(seeds, 8)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < rnn_draft_workspace(B, gamma, V, r)) return DSPARK_ERR_WORKSPACE;
  RnnDraftArgs a = {};
  a.U = U;
  a.W1 = W1;
  a.W2 = W2;
  a.Wp = Wp;
  a.hp = hp;
  a.x0 = x0;
  a.seeds = seeds;
  a.round = round;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.r = r;
  a.temperature = temperature;
  a.tokens = draft_tokens;
  a.prob = draft_prob;
  a.lse = draft_lse;
  a.e_out = e_out;
  a.ws = workspace;
  return from_hip(launch_rnn_draft(a, stream));
}

dspark_status dspark_verify(const float* U, const void* W1, const void* W2, const void* W2T, dspark_dtype wdtype,
                            const int32_t* x0,
                            const int32_t* draft_tokens, const float* draft_prob, const float* draft_rows,
                            const float* target_logits, const int32_t* lengths, int B, int gamma, int V, int r,
                            float temperature,
                            const uint64_t* seeds, uint64_t round, int32_t* accept_len, int32_t* out_tokens,
                            float* accept_prob, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(enum_value(wdtype))) return DSPARK_ERR_UNSUPPORTED;
  if (!sizes_ok(B, gamma, V, r) || !temp_ok(temperature)) return DSPARK_ERR_INVALID_ARGUMENT;
  const bool greedy = temperature == 0.0f;
  if (!req(x0, 4) || !req(draft_tokens, 4) || !req(target_logits, 16) || !req(accept_len, 4) ||
      !req(out_tokens, 4) || !opt(accept_prob, 4) || !opt(lengths, 4) || !req(workspace, 16))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (!greedy && (!req(U, 16) || !req(W1, 16) || !req(W2, 16) || !opt(W2T, 16) || !req(draft_prob, 4) ||
                  !opt(draft_rows, 4) || !req(seeds, 8)))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < verify_workspace(B, gamma, V, r)) return DSPARK_ERR_WORKSPACE;
  VerifyArgs a = {};
  a.U = U;
  a.W1 = W1;
  a.W2 = W2;
  a.W2T = greedy ? nullptr : W2T;
  a.x0 = x0;
  a.draft_tokens = draft_tokens;
  a.draft_prob = draft_prob;
  a.target = target_logits;
  a.seeds = seeds;
  a.round = round;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.r = r;
  a.temperature = temperature;
  a.accept_len = accept_len;
  a.out_tokens = out_tokens;
  a.accept_prob = accept_prob;
  a.lengths = lengths;
  a.E = greedy ? nullptr : draft_rows;
  a.ws = workspace;
  return from_hip(launch_verify(a, wdtype == DSPARK_BF16, stream));
}

dspark_status dspark_confidence(const float* h, const float* w, const void* W1, dspark_dtype wdtype,
                                const int32_t* x0, const int32_t* draft_tokens, const float* sts, int B, int gamma,
                                int d, int V, int r, float* conf, hipStream_t stream) {
  if (!dtype_ok(enum_value(wdtype))) return DSPARK_ERR_UNSUPPORTED;
  if (!sizes_ok(B, gamma, V, r) || d < 1 || d > (1 << 20)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!req(h, 16) || !req(w, 16) || !req(W1, 16) || !req(x0, 4) || !req(draft_tokens, 4) || !opt(sts, 4) ||
      !req(conf, 4))
    return DSPARK_ERR_INVALID_ARGUMENT;
  ConfArgs a = {};
  a.h = h;
  a.w = w;
  a.W1 = W1;
  a.x0 = x0;
  a.tokens = draft_tokens;
  a.sts = sts;
  a.B = B;
  a.gamma = gamma;
  a.d = d;
  a.V = V;
  a.r = r;
  a.conf = conf;
  return from_hip(launch_confidence(a, wdtype == DSPARK_BF16, stream));
}

dspark_status dspark_schedule(const float* survival, const double* sps, int sps_len, int B, int gamma,
                              dspark_schedule_mode mode, const int32_t* capacity_in, int32_t* capacity_out,
                              int32_t* lengths, double* theta, hipStream_t stream) {
  if (B < 1 || gamma < 1 || gamma > kMaxGamma || (long long)B * gamma > kScheduleMax) return DSPARK_ERR_INVALID_ARGUMENT;
  if ((long long)sps_len < (long long)B * (gamma + 1) + 1) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!req(survival, 4) || !req(sps, 8) || !req(lengths, 4) || !opt(theta, 8)) return DSPARK_ERR_INVALID_ARGUMENT;
  const int m = enum_value(mode);
  if (m != DSPARK_SCHEDULE_EARLY_STOP && m != DSPARK_SCHEDULE_CAPACITY && m != DSPARK_SCHEDULE_TOP_K)
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (mode == DSPARK_SCHEDULE_TOP_K && !req(capacity_in, 4)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!opt(capacity_out, 4)) return DSPARK_ERR_INVALID_ARGUMENT;
  return from_hip(launch_schedule(survival, sps, B, gamma, (int)mode, capacity_in,
                                  mode == DSPARK_SCHEDULE_CAPACITY ? capacity_out : nullptr, lengths, theta, stream));
}

dspark_status dspark_transpose_w2(const void* W2, dspark_dtype wdtype, int r, int V, void* W2T, hipStream_t stream) {
  if (!dtype_ok(enum_value(wdtype))) return DSPARK_ERR_UNSUPPORTED;
  if (!sizes_ok(1, 1, V, r) || !req(W2, 16) || !req(W2T, 16) || W2 == W2T) return DSPARK_ERR_INVALID_ARGUMENT;
  return from_hip(launch_transpose_w2(W2, wdtype == DSPARK_BF16, r, V, W2T, stream));
}

dspark_status dspark_survival(const float* U, const void* W1, const void* W2, dspark_dtype wdtype, const int32_t* x0,
                              const int32_t* draft_tokens, const float* draft_lse, const float* draft_rows,
                              const float* target_logits, const float* conf, int B, int gamma, int V, int r,
                              float temperature, float* c_star,
                              float* survival, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!req(survival, 4)) return DSPARK_ERR_INVALID_ARGUMENT;
  SurvivalArgs a = {};
  a.B = B;
  a.gamma = gamma;
  a.survival = survival;
  if (conf) {
    if (B < 1 || B > kMaxB || gamma < 1 || gamma > kMaxGamma || !aligned(conf, 4))
      return DSPARK_ERR_INVALID_ARGUMENT;
    a.conf = conf;
    return from_hip(launch_survival(a, false, stream));
  }
  if (!dtype_ok(enum_value(wdtype))) return DSPARK_ERR_UNSUPPORTED;
  if (!sizes_ok(B, gamma, V, r) || !temp_ok(temperature)) return DSPARK_ERR_INVALID_ARGUMENT;
  const bool greedy = temperature == 0.0f;
  if (!req(x0, 4) || !req(draft_tokens, 4) || !req(target_logits, 16) || !opt(c_star, 4) || !req(workspace, 16))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (!greedy && (!req(U, 16) || !req(W1, 16) || !req(W2, 16) || !req(draft_lse, 4) || !opt(draft_rows, 4)))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < survival_workspace(B, gamma, V, r)) return DSPARK_ERR_WORKSPACE;
  a.U = U;
  a.W1 = W1;
  a.W2 = W2;
  a.x0 = x0;
  a.draft_tokens = draft_tokens;
  a.draft_lse = draft_lse;
  a.E = greedy ? nullptr : draft_rows;
  a.target = target_logits;
  a.V = V;
  a.r = r;
  a.temperature = temperature;
  a.c_star = c_star;
  a.ws = workspace;
  return from_hip(launch_survival(a, wdtype == DSPARK_BF16, stream));
}

}  // extern "C"
