// Recording stand-ins for the kernel launchers of libdspark, so that the C ABI
// layer (csrc/api.cpp, compiled unchanged) can be exercised on the host under
// AddressSanitizer and UndefinedBehaviorSanitizer with no GPU: each launcher
// records what it was given and enqueues nothing.
#include <string.h>

#include "hostcheck.hpp"
#include "launch.hpp"

namespace hostcheck {
Record last;
int suppress_depth = 0;
}

using hostcheck::last;

namespace dspark {

// Workspace sizes in the same form as the library's (positive, growing with
// every size argument), so that the ABI's comparisons are exercised.
static size_t tiles(int V, int cols) { return ((size_t)V + cols - 1) / cols; }
size_t draft_workspace(int B, int gamma, int V, int r) { return (size_t)B * tiles(V, 128) * 8 + 16 * (size_t)B + gamma + r; }
size_t verify_workspace(int B, int gamma, int V, int r) { return (size_t)B * (gamma + 1) * tiles(V, 256) * 8 + r; }
size_t survival_workspace(int B, int gamma, int V, int r) { return (size_t)B * gamma * tiles(V, 128) * 8 + r; }
size_t rnn_draft_workspace(int B, int gamma, int V, int r) { return draft_workspace(B, gamma, V, r) + (size_t)B * gamma * 4 * r; }

hipError_t launch_draft(const DraftArgs& a, bool bf16, hipStream_t) {
  last = hostcheck::Record{};
  strcpy(last.op, "draft");
  last.B = a.B; last.gamma = a.gamma; last.V = a.V; last.r = a.r; last.T = a.temperature;
  last.round = a.round; last.bf16 = bf16; last.ws = a.ws; last.suppressed = hostcheck::suppress_depth;
  last.p[0] = a.U; last.p[1] = a.W1; last.p[2] = a.W2; last.p[3] = a.W2T; last.p[4] = a.x0;
  last.p[5] = a.seeds; last.p[6] = a.tokens; last.p[7] = a.prob; last.p[8] = a.lse; last.p[9] = a.conf;
  last.d = a.cd;
  return hipSuccess;
}

hipError_t launch_rnn_draft(const RnnDraftArgs& a, hipStream_t) {
  last = hostcheck::Record{};
  strcpy(last.op, "rnn_draft");
  last.B = a.B; last.gamma = a.gamma; last.V = a.V; last.r = a.r; last.T = a.temperature; last.ws = a.ws;
  last.p[0] = a.U; last.p[1] = a.Wp; last.p[2] = a.hp; last.p[3] = a.e_out;
  return hipSuccess;
}

hipError_t launch_verify(const VerifyArgs& a, bool bf16, hipStream_t) {
  last = hostcheck::Record{};
  strcpy(last.op, "verify");
  last.B = a.B; last.gamma = a.gamma; last.V = a.V; last.r = a.r; last.T = a.temperature; last.bf16 = bf16;
  last.ws = a.ws; last.round = a.round;
  last.p[0] = a.U; last.p[1] = a.W2T; last.p[2] = a.target; last.p[3] = a.lengths; last.p[4] = a.accept_prob;
  last.p[5] = a.E;
  return hipSuccess;
}

hipError_t launch_survival(const SurvivalArgs& a, bool, hipStream_t) {
  last = hostcheck::Record{};
  strcpy(last.op, a.conf ? "survival_conf" : "survival");
  last.B = a.B; last.gamma = a.gamma; last.V = a.V; last.r = a.r; last.ws = a.ws;
  last.p[0] = a.conf; last.p[1] = a.survival; last.p[2] = a.c_star; last.p[3] = a.E;
  return hipSuccess;
}

hipError_t launch_confidence(const ConfArgs& a, bool, hipStream_t) {
  last = hostcheck::Record{};
  strcpy(last.op, "confidence");
  last.B = a.B; last.gamma = a.gamma; last.V = a.V; last.r = a.r; last.d = a.d;
  last.p[0] = a.sts;
  return hipSuccess;
}

hipError_t launch_schedule(const float*, const double*, int B, int gamma, int mode, const int32_t* cap_in,
                           int32_t* cap_out, int32_t*, double*, hipStream_t) {
  last = hostcheck::Record{};
  strcpy(last.op, "schedule");
  last.B = B; last.gamma = gamma; last.mode = mode; last.p[0] = cap_in; last.p[1] = cap_out;
  return hipSuccess;
}

hipError_t launch_transpose_w2(const void*, bool, int r, int V, void*, hipStream_t) {
  last = hostcheck::Record{};
  strcpy(last.op, "transpose_w2");
  last.r = r; last.V = V;
  return hipSuccess;
}

hipError_t launch_markov_bias(const void*, const void*, bool, const int32_t*, int n, int V, int r, float*,
                              hipStream_t) {
  last = hostcheck::Record{};
  strcpy(last.op, "markov_bias");
  last.B = n; last.V = V; last.r = r;
  return hipSuccess;
}

size_t static_scratch_bytes() { return (size_t)32 << 20; }

static unsigned char fake_scratch[64];
hipError_t static_scratch(void** ptr) {
  *ptr = fake_scratch;
  return hipSuccess;
}

ProfSuppress::ProfSuppress() { ++hostcheck::suppress_depth; }
ProfSuppress::~ProfSuppress() { --hostcheck::suppress_depth; }

}  // namespace dspark
