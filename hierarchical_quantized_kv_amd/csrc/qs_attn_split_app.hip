// qs_attn_split_app.hip -- the attention and combine kernels of one call variant: fused append + attend over the split-upper layout (the 4-bit draft and
// verify).
#include "qs_device.h"

namespace qs {

hipError_t launch_attention_app_split(const AttnAppArgs& a, int D, bool draft, hipStream_t st) {
  return launch_attention_m<kModeAppend, kFmtSplit4>(a, D, draft, st);
}

const void* attn_fn_split_app(int D, bool draft, int bucket) {
  return attn_fn_dm<kModeAppend, false, kFmtSplit4>(D, draft, bucket);
}

}  // namespace qs
