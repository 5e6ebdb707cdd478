// qs_attn_split_host.hip -- the attention and combine kernels of one call variant: host-mode counters over the split-upper layout: the 4-bit draft and verify
// (both reading the top and middle 2-bit planes) and the 2-bit draft (top plane only).
#include "qs_device.h"

namespace qs {

hipError_t launch_attention_split(const AttnArgs& a, int D, bool draft, int fmt, hipStream_t st) {
  if (fmt == kFmtSplit2) return launch_attention_m<kModeHost, kFmtSplit2>(a, D, draft, st);
  return launch_attention_m<kModeHost, kFmtSplit4>(a, D, draft, st);
}

const void* attn_fn_split_host(int D, bool draft, int bucket, int fmt) {
  return fmt == kFmtSplit2 ? attn_fn_dm<kModeHost, false, kFmtSplit2>(D, draft, bucket)
                           : attn_fn_dm<kModeHost, false, kFmtSplit4>(D, draft, bucket);
}

}  // namespace qs
