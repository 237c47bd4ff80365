// Internal launchers of the libdspark kernels.  Host code only; arguments are
// validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

// Vocabulary columns per tile of the MFMA tile pass and of the target passes.
constexpr int kTileCols = 128;
constexpr int kTgtCols = 256;

// ceil(V / cols), in 64 bits: V may be as large as 2^31 - 1
inline int tiles_of(int V, int cols) { return (int)(((long long)V + cols - 1) / cols); }

// Which per-(row, tile) summary the tile pass writes.
enum TileMode : int {
  kModeSample = 0,   // (max l, sum 2^((l - max) * cf))      stochastic draft
  kModeGreedy = 1,   // (max l, argmax as int bits)          greedy draft
  kModeOverlap = 2,  // (sum min(p_d, p_t), 0)               analytical survival
  kModeBias = 3,     // writes the bias rows themselves       dspark_markov_bias
};

// Logical rows of the tile pass.  Row R belongs to request b = R / kper at
// block position kk = (kper == 1 ? k0 : R % kper); its previous token is x0[b]
// when kk == 0 and tokens[b * gamma + kk - 1] otherwise; its base-logit row is
// U[b][kk][:] and its target row target[b][kk][:].
struct TileArgs {
  const float* U;
  const void* W1;
  const void* W2;
  const int32_t* x0;
  const int32_t* tokens;
  const float* target;
  const float* lse_d;   // [B][gamma] natural-log normaliser of the draft (overlap mode)
  const float* lt2;     // [nrows] log2 normaliser of the target row (overlap mode)
  float2* partials;     // [nrows][ntiles]
  float* bias_out;      // [nrows][V] (bias mode)
  int nrows, kper, k0;
  int B, gamma, V, r, ntiles;
  int rows_per_group, ngroups;  // set by launch_tile_pass
  int row_begin, row_end;       // rows and tiles covered by one launch (set by launch_tile_pass)
  int tile_begin, tile_count;
  float cf;             // log2(e) / T; unused at T == 0
  const uint4* esw;     // optional: the W1 rows of the previous tokens in the ring
                        // kernel's operand layout (see ring_operand_index)
  int opnd_rows;        // 0: W1 rows of previous tokens.  n > 0: W1 is a table of operand
                        // rows, row b * gamma + kk for request b at block position kk, each
                        // of n parts of r values whose sum is the operand (generic kernel)
};

hipError_t launch_tile_pass(const TileArgs& a, int mode, bool bf16, hipStream_t s);

// Whether launch_tile_pass runs a's full tiles with the 256-row ring kernel.
bool tile_pass_uses_ring(const TileArgs& a, int mode, bool bf16);

// The ring kernel's MFMA B operand, stored ahead by the previous position's
// selection: 16-byte chunk c (k = 8c .. 8c + 7) of the W1 row of request row
// R's previous token sits at this index (in 16-byte units), so that wave w of
// row group g reads, at k-step j, 64 consecutive chunks (one per lane).
// Rows are grouped 256 to a group; r = 256 (32 chunks per row).
__host__ __device__ inline size_t ring_operand_index(int R, int c) {
  const int g = R >> 8, w = (R & 255) >> 5, n = R & 31;
  return (((size_t)g * 8 + w) * 16 + (c >> 1)) * 64 + n + 32 * (c & 1);
}

// Bytes of that buffer for `rows` rows.
inline size_t ring_operand_bytes(int rows) { return (size_t)((rows + 255) / 256) * 256 * 512; }

struct DraftArgs {
  const float* U;
  const void* W1;
  const void* W2;
  const void* W2T;   // optional [V][r] copy of W2 (enables the resident loop)
  const int32_t* x0;
  const uint64_t* seeds;
  uint64_t round;
  int B, gamma, V, r;
  float temperature;
  int32_t* tokens;
  float* prob;
  float* lse;
  // optional confidence head (conf != null): hidden states [B][gamma][cd],
  // head weights [cd + r], temperatures [gamma] (null: 1), output [B][gamma]
  const float* ch;
  const float* cw;
  const float* csts;
  int cd;
  float* conf;
  void* ws;
};

size_t draft_workspace(int B, int gamma, int V, int r);
hipError_t launch_draft(const DraftArgs& a, bool bf16, hipStream_t s);

// The device-resident draft loop (resident.hip): whether it applies to these
// arguments, its workspace, and its launch (*launched false: not enqueued,
// the caller uses the per-position launches).
bool resident_draft_applies(const DraftArgs& a, bool bf16);
size_t resident_workspace(int B, int gamma, int V, int r);
hipError_t launch_resident_draft(const DraftArgs& a, hipStream_t s, bool* launched);

// Block sampling with the RNN head (bf16 W1 and W2 only).
struct RnnDraftArgs {
  const float* U;
  const void* W1;
  const void* W2;
  const float* Wp;   // [3r][2r] recurrent and token columns of the cell projection
  const float* hp;   // [B][gamma][3r] hidden-state part of the projection
  const int32_t* x0;
  const uint64_t* seeds;
  uint64_t round;
  int B, gamma, V, r;
  float temperature;
  int32_t* tokens;
  float* prob;
  float* lse;
  float* e_out;      // optional [B][gamma][r]
  void* ws;
};

size_t rnn_draft_workspace(int B, int gamma, int V, int r);
hipError_t launch_rnn_draft(const RnnDraftArgs& a, hipStream_t s);

struct VerifyArgs {
  const float* U;
  const void* W1;
  const void* W2;
  const void* W2T;  // optional [V][r] copy of W2
  const int32_t* x0;
  const int32_t* draft_tokens;
  const float* draft_prob;
  const float* target;
  const uint64_t* seeds;
  uint64_t round;
  int B, gamma, V, r;
  float temperature;
  int32_t* accept_len;
  int32_t* out_tokens;
  float* accept_prob;
  const int32_t* lengths;  // optional [B] scheduled verification lengths (null: gamma)
  const float* E;          // optional [B][gamma][r] operand rows e_k of an RNN draft (null: W1[x_{k-1}])
  void* ws;
  double inv_t_d;  // 1 / T, filled in by launch_verify
};

size_t verify_workspace(int B, int gamma, int V, int r);
hipError_t launch_verify(const VerifyArgs& a, bool bf16, hipStream_t s);

struct SurvivalArgs {
  const float* U;
  const void* W1;
  const void* W2;
  const int32_t* x0;
  const int32_t* draft_tokens;
  const float* draft_lse;
  const float* target;
  const float* conf;
  const float* E;  // optional [B][gamma][r] operand rows e_k of an RNN draft (null: W1[x_{k-1}])
  int B, gamma, V, r;
  float temperature;
  float* c_star;
  float* survival;
  void* ws;
};

size_t survival_workspace(int B, int gamma, int V, int r);
hipError_t launch_survival(const SurvivalArgs& a, bool bf16, hipStream_t s);

// Target-row statistics (verify.hip), shared by verify and survival.
//   list mode (list != null): rows_per_req rows (block positions kk0, kk0+1,
//     ...) of each listed request b; summaries of row j go to row
//     b * orow_stride + j of tpart.
//   all mode: row R = b * gamma + kk for kk < gamma; summaries go to row R.
// Sample mode writes (max t, sum 2^((t - max) * cf)) per kTgtCols-column tile;
// greedy mode (max t, argmax as int bits).
struct TStatsArgs {
  const float* target;
  const int* list;
  const int* count;  // device count (list mode)
  int nreq;          // list mode: entries of the list buffer; request mode: requests
  int nall;          // rows in all mode
  int max_rows;      // bound on the rows of one launch (set by launch_target_stats)
  int kk0;
  int rows_per_req;  // list mode: block positions kk0, kk0+1, ... of each listed request
  int orow_stride;   // list mode: summaries of (b, row) go to row b * orow_stride + row
  int gamma, V, ntv;
  float cf;
  float2* tpart;
  const int32_t* draft_tokens;  // with tx_out: the drafted tokens [B][gamma]
  float* tx_out;                // list mode, optional: target logit of the drafted token per output row
  const int32_t* lengths;       // list mode, optional: scheduled lengths; rows past l_b + 1 are not read
};

hipError_t launch_target_stats(const TStatsArgs& a, bool greedy, int max_rows, hipStream_t s);

// Compute units of the current device (queried once per device).
int compute_units_of_device();

// Confidence head (confidence.hip).
struct ConfArgs {
  const float* h;        // [B][gamma][d] hidden states
  const float* w;        // [d + r] head weights, hidden part first
  const void* W1;        // [V][r] Markov embedding
  const int32_t* x0;     // [B]
  const int32_t* tokens; // [B][gamma] drafted tokens
  const float* sts;      // [gamma] temperatures (null: 1)
  int B, gamma, d, V, r;
  float* conf;           // [B][gamma]
};
hipError_t launch_confidence(const ConfArgs& a, bool bf16, hipStream_t s);

// Hardware-aware prefix scheduler (schedule.hip): one workgroup, at most
// kScheduleMax candidates (B * gamma).
constexpr int kScheduleMax = 16384;
constexpr int kScheduleEarlyStop = 0;  // Algorithm 1
constexpr int kScheduleCapacity = 1;   // first maximum of Theta over the whole scan
constexpr int kScheduleTopK = 2;       // the first K candidates, K given on the device
hipError_t launch_schedule(const float* survival, const double* sps, int B, int gamma, int mode,
                           const int32_t* cap_in, int32_t* cap_out, int32_t* lengths, double* theta, hipStream_t s);

hipError_t launch_transpose_w2(const void* W2, bool bf16, int r, int V, void* W2T, hipStream_t s);

hipError_t launch_markov_bias(const void* W1, const void* W2, bool bf16, const int32_t* tokens,
                              int n, int V, int r, float* out, hipStream_t s);

// Kernel kinds of the optional event timing (profile.cpp).
enum ProfKind : int {
  kProfTileSample = 0, kProfTileGreedy, kProfTileOverlap, kProfTileBias, kProfDraftSelect,
  kProfVerifyInit, kProfTargetStats, kProfVerifyDecide, kProfResidualStats, kProfResidualSelect,
  kProfSurvivalConf, kProfSurvivalTnorm, kProfSurvivalFinish, kProfSchedule, kProfConfidence, kProfRnnCell,
  kProfResidentDraft, kProfKinds
};

// Brackets the launches made during its lifetime with HIP events when timing
// is enabled (dspark_profile_enable); otherwise does nothing.
class ProfScope {
 public:
  ProfScope(hipStream_t s, int kind);
  ~ProfScope();
  // the bracketed launch did not happen: the record is kept out of the sums
  void discard();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  hipStream_t stream_;
  int index_;
};

// While one exists on the calling thread, ProfScope records nothing (no
// events are created or recorded): used by the allocation-free entry point.
class ProfSuppress {
 public:
  ProfSuppress();
  ~ProfSuppress();
  ProfSuppress(const ProfSuppress&) = delete;
  ProfSuppress& operator=(const ProfSuppress&) = delete;
};

// The library's static device scratch array (noalloc.hip): its size, and its
// address on the current device (looked up once per device).
size_t static_scratch_bytes();
hipError_t static_scratch(void** ptr);

// Round a byte count up to a 256-byte boundary (workspace carving).
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace dspark
