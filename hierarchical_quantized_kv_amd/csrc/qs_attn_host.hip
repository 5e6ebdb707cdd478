// qs_attn_host.hip -- the attention and combine kernels of one call variant: host-mode counters (qs_attend_draft / qs_attend_verify).
#include "qs_device.h"

namespace qs {

hipError_t launch_attention(const AttnArgs& a, int D, bool draft, hipStream_t st) {
  return launch_attention_m<kModeHost>(a, D, draft, st);
}

const void* attn_fn_host(int D, bool draft, int bucket, bool meta16) {
  return meta16 ? attn_fn_dm<kModeHost, true>(D, draft, bucket) : attn_fn_dm<kModeHost, false>(D, draft, bucket);
}

}  // namespace qs
