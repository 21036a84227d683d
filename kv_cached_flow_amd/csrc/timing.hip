// Optional per-kernel-class timing with HIP events (off by default).  When
// enabled, every launch records an event pair on its own stream and adds its
// algorithmic work (bytes moved / flops the method needs, not counters).
#include <mutex>
#include <vector>

#include "wam_internal.h"

namespace wam {

namespace {
struct Rec {
  int cls;
  hipEvent_t a, b;
  double bytes, flops;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t get_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

const char* kNames[KC_COUNT] = {"gemm_big",    "gemm_skinny", "gemm_simple", "attn_prefill",
                                "attn_action", "attn_merge",  "rmsnorm",     "embed",
                                "fuse_kv",     "quant_kv",    "misc"};
}  // namespace

bool timing_on() { return g_on; }

TimingScope::TimingScope(hipStream_t s, int cls, double bytes, double flops)
    : s_(s), cls_(cls), bytes_(bytes), flops_(flops), a_(nullptr) {
  if (!g_on) return;
  std::lock_guard<std::mutex> lk(g_mu);
  a_ = get_event();
  if (a_) hipEventRecord((hipEvent_t)a_, s_);
}

TimingScope::~TimingScope() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t b = get_event();
  if (!b) return;
  hipEventRecord(b, s_);
  g_recs.push_back(Rec{cls_, (hipEvent_t)a_, b, bytes_, flops_});
}

}  // namespace wam

extern "C" int wam_timing(int enable) {
  using namespace wam;
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_recs) {
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  g_on = enable != 0;
  return WAM_OK;
}

extern "C" int wam_timing_report(wam_kernel_stat* out, int max) {
  using namespace wam;
  std::lock_guard<std::mutex> lk(g_mu);
  wam_kernel_stat acc[KC_COUNT];
  for (int c = 0; c < KC_COUNT; c++) {
    memset(&acc[c], 0, sizeof acc[c]);
    strncpy(acc[c].name, kNames[c], sizeof acc[c].name - 1);
  }
  for (auto& r : g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return WAM_E_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return WAM_E_HIP;
    acc[r.cls].launches++;
    acc[r.cls].ms += ms;
    acc[r.cls].bytes += r.bytes;
    acc[r.cls].flops += r.flops;
  }
  int n = 0;
  for (int c = 0; c < KC_COUNT && n < max; c++)
    if (acc[c].launches) out[n++] = acc[c];
  return n;
}
