// qs_attn_dev.hip -- the attention and combine kernels of one call variant: device-mode counters (qs_attend_draft_dev / qs_attend_verify_dev).
#include "qs_device.h"

namespace qs {

hipError_t launch_attention_dev(const AttnDevArgs& a, int D, bool draft, hipStream_t st) {
  return launch_attention_m<kModeDev>(a, D, draft, st);
}

const void* attn_fn_dev(int D, bool draft, int bucket, bool meta16) {
  return meta16 ? attn_fn_dm<kModeDev, true>(D, draft, bucket) : attn_fn_dm<kModeDev, false>(D, draft, bucket);
}

}  // namespace qs
