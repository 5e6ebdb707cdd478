// qs_attn_app.hip -- the attention and combine kernels of one call variant: fused append + attend (qs_append_attend_draft / qs_append_attend_verify).
#include "qs_device.h"

namespace qs {

hipError_t launch_attention_app(const AttnAppArgs& a, int D, bool draft, hipStream_t st) {
  return launch_attention_m<kModeAppend>(a, D, draft, st);
}

const void* attn_fn_app(int D, bool draft, int bucket, bool meta16) {
  return meta16 ? attn_fn_dm<kModeAppend, true>(D, draft, bucket) : attn_fn_dm<kModeAppend, false>(D, draft, bucket);
}

}  // namespace qs
