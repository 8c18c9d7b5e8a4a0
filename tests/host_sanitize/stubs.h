// The launch records of the host-only stub launchers (stub_launchers.cpp).
#pragma once

#include "../../decode_attention_folded_amd/csrc/check.h"
#include "../../decode_attention_folded_amd/csrc/kernels.h"

namespace da {

struct StubRecord {
  enum Kind { kNone, kAttn, kMeta, kScore, kTopk, kRepeat, kCheck, kCalibration };
  Kind last = kNone;
  long launches = 0;
  AttnLaunch attn{};
  MetaLaunch meta{};
  ScoreLaunch score{};
  ScoreLaunch topk{};
  RepeatLaunch repeat{};
};

extern StubRecord g_stub;

}  // namespace da
