// Library-wide entry points: version, status strings, workspace sizes, timing.
#include "common.h"

namespace gq {

size_t hessian_workspace_bytes(int64_t d, int64_t n_rows, int64_t batch, int dtype);
size_t prepare_workspace_bytes(int64_t d, int64_t batch);
size_t quantize_workspace_bytes(const gptq_params* p, int64_t d_out, int64_t d_in, int64_t batch);
size_t w4a16_workspace_bytes(int64_t M, int64_t d_in, int64_t d_out);
size_t abs_workspace_bytes(int64_t d, int64_t n_rows);
size_t awq_search_workspace_bytes(int64_t d_out, int64_t d_in, int64_t n_s, int64_t n_alpha);
size_t forward_workspace_bytes(int64_t n_tok, int64_t d_in, int64_t d_out);

// ---------------------------------------------------------------- timing state
namespace {
struct TimingState {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[kTimeKinds];
  std::vector<hipEvent_t> pool;
};
TimingState g_timing;

hipEvent_t take_event() {
  if (!g_timing.pool.empty()) {
    hipEvent_t e = g_timing.pool.back();
    g_timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

TimedScope::TimedScope(int k, hipStream_t s) : kind(k), stream(s) {
  if (!g_timing.on || k < 0 || k >= kTimeKinds) return;   // k < 0: a launch that is never timed
  start = take_event();
  if (start) hipEventRecord(start, stream);
}

TimedScope::~TimedScope() {
  if (!start) return;
  hipEvent_t stop = take_event();
  if (!stop) return;
  hipEventRecord(stop, stream);
  g_timing.ev[kind].emplace_back(start, stop);
}

}  // namespace gq

using namespace gq;

extern "C" int32_t gptq_abi_version(void) { return GPTQ_ABI_VERSION; }

extern "C" const char* gptq_status_string(int32_t s) {
  switch (s) {
    case GPTQ_OK: return "ok";
    case GPTQ_EINVAL: return "invalid argument";
    case GPTQ_ENOTPD: return "damped Hessian is not positive definite";
    case GPTQ_EHIP: return "HIP runtime error";
    case GPTQ_EUNSUPPORTED: return "unsupported configuration";
    case GPTQ_ENOMEM: return "workspace too small";
    default: return "unknown status";
  }
}

bool gq_params_ok(const gptq_params* p, int64_t d_in);

extern "C" gptq_status gptq_workspace_size(int32_t op, const gptq_params* p, int64_t d_out, int64_t d_in,
                                           int64_t n_rows, int64_t batch, size_t* bytes_out) {
  GQ_CHECK_ARG(bytes_out != nullptr);
  GQ_CHECK_ARG(d_in >= 1 && batch >= 1);
  switch (op) {
    case GPTQ_OP_HESSIAN:
      GQ_CHECK_ARG(n_rows >= 0);
      // the bf16/fp16 path needs the larger workspace; report that one
      *bytes_out = std::max(hessian_workspace_bytes(d_in, n_rows, batch, GPTQ_BF16),
                            hessian_workspace_bytes(d_in, n_rows, batch, GPTQ_F32));
      return GPTQ_OK;
    case GPTQ_OP_PREPARE:
      *bytes_out = prepare_workspace_bytes(d_in, batch);
      return GPTQ_OK;
    case GPTQ_OP_QUANTIZE:
      GQ_CHECK_ARG(p != nullptr && d_out >= 1);
      GQ_CHECK_ARG(gq_params_ok(p, d_in));
      *bytes_out = quantize_workspace_bytes(p, d_out, d_in, batch);
      return GPTQ_OK;
    case GPTQ_OP_W4A16:
      GQ_CHECK_ARG(d_out >= 1 && n_rows >= 1);
      *bytes_out = w4a16_workspace_bytes(n_rows, d_in, d_out);
      return GPTQ_OK;
    case GPTQ_OP_ABS:
      GQ_CHECK_ARG(n_rows >= 0);
      *bytes_out = abs_workspace_bytes(d_in, n_rows);
      return GPTQ_OK;
    case GPTQ_OP_AWQ_SEARCH:
      GQ_CHECK_ARG(d_out >= 1 && n_rows >= 1);
      *bytes_out = awq_search_workspace_bytes(d_out, d_in, n_rows, batch);
      return GPTQ_OK;
    case GPTQ_OP_FORWARD:
      GQ_CHECK_ARG(d_out >= 1 && n_rows >= 0);
      *bytes_out = forward_workspace_bytes(n_rows, d_in, d_out);
      return GPTQ_OK;
    default:
      return GPTQ_EINVAL;
  }
}

extern "C" gptq_status gptq_timing_enable(int32_t on) {
  g_timing.on = on != 0;
  return GPTQ_OK;
}

extern "C" gptq_status gptq_timing_reset(void) {
  for (auto& v : g_timing.ev) {
    for (auto& pr : v) {
      g_timing.pool.push_back(pr.first);
      g_timing.pool.push_back(pr.second);
    }
    v.clear();
  }
  return GPTQ_OK;
}

extern "C" gptq_status gptq_timing_read(int32_t kind, double* total_ms, int64_t* launches) {
  GQ_CHECK_ARG(kind >= 0 && kind < kTimeKinds && total_ms && launches);
  double t = 0.0;
  for (auto& pr : g_timing.ev[kind]) {
    GQ_HIP(hipEventSynchronize(pr.second));
    float ms = 0.f;
    GQ_HIP(hipEventElapsedTime(&ms, pr.first, pr.second));
    t += ms;
  }
  *total_ms = t;
  *launches = (int64_t)g_timing.ev[kind].size();
  return GPTQ_OK;
}
