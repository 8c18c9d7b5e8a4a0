// Folded-GQA decode attention (attention_impl.h) over pages that the kernel
// selects itself from the page scores: the instantiations for every
// items-per-thread width of the in-kernel top-K, in a translation unit of
// their own so the two halves compile in parallel.

#include "attention_impl.h"

namespace da {
namespace {

// Items per thread of the in-kernel top-K: the score row in 256-thread blocks.
template <int D, int G, bool PAGED>
int launch_select(const AttnLaunch& a, hipStream_t s) {
  const int P = a.sel_row;
  if (P <= kTopkThreads * 8) return launch_one<D, G, PAGED, true, 8>(a, s);
  if (P <= kTopkThreads * 16) return launch_one<D, G, PAGED, true, 16>(a, s);
  if (P <= kTopkThreads * 32) return launch_one<D, G, PAGED, true, 32>(a, s);
  if (P <= kTopkThreads * 64) return launch_one<D, G, PAGED, true, 64>(a, s);
  return (int)hipErrorInvalidValue;
}

template <int D, int G>
int launch_select_dg(const AttnLaunch& a, hipStream_t s) {
  return a.page_table != nullptr ? launch_select<D, G, true>(a, s)
                                 : launch_select<D, G, false>(a, s);
}

template <int D>
int launch_select_d(const AttnLaunch& a, hipStream_t s) {
  switch (a.group) {
    case 1: return launch_select_dg<D, 1>(a, s);
    case 2: return launch_select_dg<D, 2>(a, s);
    case 4: return launch_select_dg<D, 4>(a, s);
    case 8: return launch_select_dg<D, 8>(a, s);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

int launch_select_attention(const AttnLaunch& a, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.head_dim == 64) return launch_select_d<64>(a, s);
  if (a.head_dim == 128) return launch_select_d<128>(a, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace da
