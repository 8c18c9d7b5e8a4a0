// Folded-GQA decode attention (attention_impl.h): the instantiations for a
// contiguous or paged cache, dense or over a given list of chosen pages, and
// the launch entry used by the C ABI.

#include "attention_impl.h"

namespace da {
namespace {

template <int D, int G>
int launch_dg(const AttnLaunch& a, hipStream_t s) {
  const bool paged = a.page_table != nullptr;
  const bool sparse = a.page_idx != nullptr;
  if (paged)
    return sparse ? launch_one<D, G, true, true, 0>(a, s) : launch_one<D, G, true, false, 0>(a, s);
  return sparse ? launch_one<D, G, false, true, 0>(a, s) : launch_one<D, G, false, false, 0>(a, s);
}

template <int D>
int launch_d(const AttnLaunch& a, hipStream_t s) {
  switch (a.group) {
    case 1: return launch_dg<D, 1>(a, s);
    case 2: return launch_dg<D, 2>(a, s);
    case 4: return launch_dg<D, 4>(a, s);
    case 8: return launch_dg<D, 8>(a, s);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

int keys_per_tile(int, int) { return kTileKeys; }

int max_tiles_per_split(bool page_list) {
  return page_list ? kMaxTilesPerSplit : kMaxTilesPerSplitContiguous;
}

int launch_decode(const AttnLaunch& a, void* stream) {
  if (a.sel_scores != nullptr) return launch_select_attention(a, stream);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.head_dim == 64) return launch_d<64>(a, s);
  if (a.head_dim == 128) return launch_d<128>(a, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace da
