// Host-only stand-ins for the kernel launchers of kernels.h, so that the C ABI
// layer (api.cpp) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven on a machine without a GPU.  Each
// stub records the launch it was asked for and enqueues nothing; the plan
// constants are the device code's (tests/test_host_sanitize.py checks the
// workspace sizes they lead to against the real library).

#include <stddef.h>
#include <stdint.h>

#include "stubs.h"

namespace da {

StubRecord g_stub;

int keys_per_tile(int, int) { return 16; }
int max_tiles_per_split(bool page_list) { return page_list ? 160 : 512; }
int topk_max_pages() { return 256 * 64; }
size_t noalloc_scratch_bytes() { return size_t(32) << 20; }
int noalloc_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(uintptr_t(0x7f0000000000ull));  // never dereferenced
  return 0;
}

int launch_decode(const AttnLaunch& p, void*) {
  g_stub.attn = p;
  g_stub.last = StubRecord::kAttn;
  ++g_stub.launches;
  return 0;
}
int launch_select_attention(const AttnLaunch& p, void* s) { return launch_decode(p, s); }
int launch_meta_append(const MetaLaunch& p, void*) {
  g_stub.meta = p;
  g_stub.last = StubRecord::kMeta;
  ++g_stub.launches;
  return 0;
}
int launch_score_topk(const ScoreLaunch& p, void*) {
  g_stub.score = p;
  g_stub.last = StubRecord::kScore;
  ++g_stub.launches;
  return 0;
}
int launch_topk_only(const ScoreLaunch& p, void*) {
  g_stub.topk = p;
  g_stub.last = StubRecord::kTopk;
  ++g_stub.launches;
  return 0;
}
int launch_repeat_kv(const RepeatLaunch& p, void*) {
  g_stub.repeat = p;
  g_stub.last = StubRecord::kRepeat;
  ++g_stub.launches;
  return 0;
}
int repeat_kv_rows_per_workgroup() { return 64; }
int launch_check(const CheckLaunch&, void*) {
  g_stub.last = StubRecord::kCheck;
  ++g_stub.launches;
  return 0;
}
int launch_read_calibration(const void*, uint64_t, uint32_t*, void*) {
  g_stub.last = StubRecord::kCalibration;
  ++g_stub.launches;
  return 0;
}

}  // namespace da
